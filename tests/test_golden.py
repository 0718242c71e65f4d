"""Hand-worked examples (tests/golden/worked_examples.json) against the oracle
on the CPU and against the HIP kernels on the GPU.

The pages print no worked example with numbers; the fixture's values are
derived by hand from the equations they state (the fixture cites each one)
in exact dyadic arithmetic, so the oracle must reproduce them exactly.  On
the GPU the d = 2 (and d = 1) examples are embedded in d = 64 / 128 heads
whose other channels are zero, which changes no result: every kernel path
(float32 vector ALU, bf16 MFMA at each block level, packed, channel-wise,
backward, decode) must return the worked values.  All of them are exact in
bf16 as well; the kernels form decay powers as 2^(n log2 lambda) in float32,
so the GPU comparison allows float32 rounding.
"""
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
    EXAMPLES = {e["name"]: e for e in json.load(f)["examples"]}


def arr(x, *lead):
    a = np.asarray(x, np.float64)
    return a.reshape(lead + a.shape)


# ------------------------------------------------------------- oracle (CPU)


def test_oracle_recurrence():
    e = EXAMPLES["recurrence_d2_n3_lambda_half"]
    q, k, v = (arr(e[n], 1, 1) for n in "qkv")
    lam = np.array([e["lambda"]], np.float32)
    out, fin, _ = oracle.fwd(q, k, v, lam)
    assert np.array_equal(out[0, 0], arr(e["out"])) and np.array_equal(fin[0, 0],
                                                                       arr(e["final_state"]))
    # the quadratic (left-product) form and the decode steps give the same numbers
    out_b, fin_b = oracle.bruteforce(q, k, v, lam)
    assert np.array_equal(out_b[0, 0], arr(e["out"])) and np.array_equal(fin_b[0, 0],
                                                                         arr(e["final_state"]))
    state = np.zeros((1, 1, 2, 2))
    for t in range(3):
        o, _ = oracle.decode(q[:, :, t], k[:, :, t], v[:, :, t], lam, state)
        assert np.array_equal(o[0, 0], arr(e["out"])[t])
    assert np.array_equal(state[0, 0], arr(e["final_state"]))


def test_oracle_initial_state():
    e = EXAMPLES["recurrence_with_initial_state"]
    q, k, v = (arr(e[n], 1, 1) for n in "qkv")
    lam = np.array([e["lambda"]], np.float32)
    out, fin, _ = oracle.fwd(q, k, v, lam, init=arr(e["init"], 1, 1))
    assert np.array_equal(out[0, 0], arr(e["out"]))
    assert np.array_equal(fin[0, 0], arr(e["final_state"]))


def test_oracle_packed():
    e = EXAMPLES["packed_two_sequences"]
    q, k, v = (arr(e[n], 1) for n in "qkv")
    lam = np.array([e["lambda"]], np.float32)
    out, fins, _ = oracle.fwd_varlen(q, k, v, lam, np.array(e["cu_seqlens"], np.int32))
    assert np.array_equal(out[0], arr(e["out"]))
    assert np.array_equal(fins[:, 0], arr(e["final_states"]))


def test_oracle_channel_wise():
    e = EXAMPLES["channel_wise_decay"]
    q, k, v = (arr(e[n], 1, 1) for n in "qkv")
    out, fin = oracle.fwd_chdecay(q, k, v, arr(e["alpha"], 1))
    assert np.array_equal(out[0, 0], arr(e["out"]))
    assert np.array_equal(fin[0, 0], arr(e["final_state"]))


def test_oracle_backward():
    e = EXAMPLES["backward_d1_n2"]
    q, k, v, do = (arr(e[n], 1, 1) for n in ("q", "k", "v", "dout"))
    lam = np.array([e["lambda"]], np.float32)
    dq, dk, dv, dinit = oracle.bwd(q, k, v, lam, do, dfin=arr(e["dfin"], 1, 1),
                                   init=arr(e["init"], 1, 1))
    for got, name in ((dq, "dq"), (dk, "dk"), (dv, "dv"), (dinit, "dinit")):
        assert np.array_equal(got[0, 0], arr(e[name])), name


# ------------------------------------------------------------- HIP path (GPU)


def embed_rows(x, d):
    """[N, d0] rows into [N, d] with zero channels beyond d0."""
    x = np.asarray(x, np.float32)
    out = np.zeros((x.shape[0], d), np.float32)
    out[:, :x.shape[1]] = x
    return out


def embed_state(s, d):
    s = np.asarray(s, np.float32)
    out = np.zeros((d, d), np.float32)
    out[:s.shape[0], :s.shape[1]] = s
    return out


def close(got, ref, tol=1e-6):
    ref = np.asarray(ref, np.float64)
    got = np.asarray(got, np.float64)[tuple(slice(0, n) for n in ref.shape)]
    return np.abs(got - ref).max() <= tol * max(1.0, np.abs(ref).max())


def zero_beyond(got, shape):
    """Every entry outside the embedded block is zero."""
    g = np.array(got, np.float64, copy=True)
    g[tuple(slice(0, n) for n in shape)] = 0.0
    return not np.any(g)


PATHS = [("fp32", 64, 128), ("bf16", 128, 128), ("bf16", 128, 64), ("bf16", 128, 32)]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,d,block", PATHS)
@pytest.mark.parametrize("name", ["recurrence_d2_n3_lambda_half",
                                  "recurrence_with_initial_state"])
def test_gpu_worked_recurrence(name, dtype, d, block):
    import torch
    import linear_attention_lightning_amd as la
    e = EXAMPLES[name]
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    q, k, v = (torch.from_numpy(embed_rows(e[n], d)).reshape(1, 1, 3, d).to(tdt).cuda()
               for n in "qkv")
    lam = torch.tensor([e["lambda"]], dtype=torch.float32).cuda()
    init = None
    if "init" in e:
        init = torch.from_numpy(embed_state(e["init"], d)).reshape(1, 1, d, d).cuda()
    out, fin = la.lightning_attn_fwd(q, k, v, lam, block=block, init_state=init)
    torch.cuda.synchronize()
    o = out[0, 0].float().cpu().numpy()
    s = fin[0, 0].cpu().numpy()
    assert close(o, e["out"]) and zero_beyond(o, (3, 2)), o[:, :2]
    assert close(s, e["final_state"]) and zero_beyond(s, (2, 2)), s[:2, :2]
    # the same tokens as three decode steps from the initial state
    st = init.clone() if init is not None else torch.zeros((1, 1, d, d), device="cuda")
    for t in range(3):
        o_t = la.lightning_attn_decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                       v[:, :, t].contiguous(), lam, st)
        torch.cuda.synchronize()
        assert close(o_t[0, 0].float().cpu().numpy(), e["out"][t])
    assert close(st[0, 0].cpu().numpy(), e["final_state"])


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,d,block", PATHS)
def test_gpu_worked_packed(dtype, d, block):
    import torch
    import linear_attention_lightning_amd as la
    e = EXAMPLES["packed_two_sequences"]
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    q, k, v = (torch.from_numpy(embed_rows(e[n], d)).reshape(1, 3, d).to(tdt).cuda()
               for n in "qkv")
    lam = torch.tensor([e["lambda"]], dtype=torch.float32).cuda()
    cu = torch.tensor(e["cu_seqlens"], dtype=torch.int32).cuda()
    for seg in (0, la.LA_SEGMENT_PER_SEQUENCE, 1):
        out, fins = la.lightning_attn_fwd_varlen(q, k, v, lam, cu, block=block,
                                                 segment_tokens=seg)
        torch.cuda.synchronize()
        assert close(out[0].float().cpu().numpy(), e["out"]), seg
        for j, ref in enumerate(e["final_states"]):
            assert close(fins[j, 0].cpu().numpy(), ref), (seg, j)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,d", [("fp32", 64), ("bf16", 128)])
def test_gpu_worked_channel_wise(dtype, d):
    import torch
    import linear_attention_lightning_amd as la
    e = EXAMPLES["channel_wise_decay"]
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    q, k, v = (torch.from_numpy(embed_rows(e[n], d)).reshape(1, 1, 3, d).to(tdt).cuda()
               for n in "qkv")
    alpha = np.ones((1, d), np.float32)  # the zero channels' decay does not matter
    alpha[0, :2] = e["alpha"]
    out, fin = la.lightning_attn_fwd_chdecay(q, k, v, torch.from_numpy(alpha).cuda())
    torch.cuda.synchronize()
    assert close(out[0, 0].float().cpu().numpy(), e["out"])
    assert close(fin[0, 0].cpu().numpy(), e["final_state"])


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,d", [("fp32", 64), ("bf16", 128)])
def test_gpu_worked_backward(dtype, d):
    import torch
    import linear_attention_lightning_amd as la
    e = EXAMPLES["backward_d1_n2"]
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    q, k, v, do = (torch.from_numpy(embed_rows(e[n], d)).reshape(1, 1, 2, d).to(tdt).cuda()
                   for n in ("q", "k", "v", "dout"))
    lam = torch.tensor([e["lambda"]], dtype=torch.float32).cuda()
    init = torch.from_numpy(embed_state(e["init"], d)).reshape(1, 1, d, d).cuda()
    dfin = torch.from_numpy(embed_state(e["dfin"], d)).reshape(1, 1, d, d).cuda()
    dq, dk, dv, dinit = la.lightning_attn_bwd(q, k, v, lam, do, dfinal=dfin, init_state=init)
    torch.cuda.synchronize()
    for got, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        g = got[0, 0].float().cpu().numpy()
        assert close(g, e[name]), (name, g[:, :1])
    assert close(dinit[0, 0].cpu().numpy(), e["dinit"])
