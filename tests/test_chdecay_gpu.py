"""GPU parity of the channel-wise decay prefill (lightning_attn_fwd_chdecay)
against the CPU oracle's channel-wise recurrence (oracle.fwd_chdecay, pinned
to the per-channel decomposition of the decayed left product).

Bar as for the scalar decay: max |x - x_ref| / max |x_ref| <= 1e-4 for
float32 inputs, <= 2e-2 for bf16 inputs, for outputs and final states.
"""
import sys

import numpy as np
import pytest

import oracle
import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import inputs
from parity_util import ORACLE_CACHE, whole_rel_err

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def torch_mod():
    import torch
    return torch


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.abs(b).max() if b.size else 0.0
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0)) if a.size else 0.0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    torch = torch_mod()
    return t.detach().to(torch.float32).cpu().numpy()


def run_ch_case(B, H, N, d, dtype, seed, seg=0, with_init=True, alpha=None, token_major=False,
                block=128):
    torch = torch_mod()
    say("case chdecay B=%d H=%d N=%d d=%d %s seg=%d init=%s token_major=%s"
        % (B, H, N, d, dtype, seg, with_init, token_major))
    q, k, v = inputs.host_qkv((B, H, N, d), seed, dtype=dtype)
    alpha = inputs.chdecay_schedule(H, d, seed + 1) if alpha is None else alpha
    init = inputs.host_state((B, H, d, d), seed + 2) if with_init else None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tq, tk, tv = (torch.from_numpy(x).cuda().to(tdt) for x in (q, k, v))
    layout = la.LA_HEAD_MAJOR
    if token_major:
        tq, tk, tv = (t.transpose(1, 2).contiguous() for t in (tq, tk, tv))
        layout = la.LA_TOKEN_MAJOR
    out = torch.full_like(tq, float("nan"))
    out, fin = la.lightning_attn_fwd_chdecay(
        tq, tk, tv, torch.from_numpy(alpha).cuda(), layout=layout, block=block,
        init_state=None if init is None else torch.from_numpy(init).cuda(), segment_tokens=seg,
        out=out)
    torch.cuda.synchronize()
    if token_major:
        out = out.transpose(1, 2)
    o_ref, f_ref = oracle.fwd_chdecay(q, k, v, alpha, init=init)
    ho = host(out)
    assert np.isfinite(ho).all()
    eo, ef = rel_err(ho, o_ref), rel_err(host(fin), f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL[dtype] and ef <= TOL[dtype], (eo, ef)
    return out, fin


def test_chdecay_tiny_fp32():
    run_ch_case(1, 2, 256, 64, "fp32", seed=600, block=64)


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "bf16"), (128, "fp32"), (64, "fp32")])
@pytest.mark.parametrize("seg", [0, 100, 640, la.LA_SEGMENT_PER_SEQUENCE])
def test_chdecay_segments(d, dtype, seg):
    """Segment cuts that hand per-channel states on (the scan weighs every
    state row by its own channel's decay)."""
    run_ch_case(2, 3, 1000, d, dtype, seed=610 + d, seg=seg)


@pytest.mark.parametrize("N", [1, 31, 32, 33, 300])
def test_chdecay_ragged(N):
    run_ch_case(2, 2, N, 128, "bf16", seed=620 + N, seg=64)


def small_alpha(H, d, seed):
    """Per-channel decays with small values: head 1 has every third channel
    at 0.05, head 2 every other channel at 0.01, head 3 every channel at 1e-3
    but channel 0 at 1, head 4 channels from exactly 1/8 (the smallest decay
    the MFMA output pass takes: its largest factor alpha^-32 is 2^96) to 1,
    head 5 one channel just below 1/8; heads 0 and 6+ from the schedule."""
    alpha = inputs.chdecay_schedule(H, d, seed).copy()
    alpha[1, ::3] = 0.05
    alpha[2, ::2] = 0.01
    alpha[3, :] = 1e-3
    alpha[3, 0] = 1.0
    alpha[4] = np.linspace(0.125, 1.0, d)
    alpha[5, 5] = 0.1249
    return alpha.astype(np.float32)


@pytest.mark.parametrize("seg", [0, 256, la.LA_SEGMENT_PER_SEQUENCE])
def test_chdecay_small_alpha(seg):
    """Heads whose smallest decay is below 1/8 (0.05, 0.01, 1e-3, 0.1249) run
    their output pass on the vector-ALU kernel beside the MFMA heads (1/8
    exactly and the schedule's): every output finite and within the bar, with
    segment cuts (the local-state pass and the scan take every head) and
    without."""
    run_ch_case(1, 7, 1500, 128, "bf16", seed=650, seg=seg, alpha=small_alpha(7, 128, 651))


def test_chdecay_small_alpha_varlen():
    run_ch_varlen_case([300, 0, 1000, 7, 0, 2000, 129], 7, 128, "bf16", seed=660, seg=200,
                       alpha=small_alpha(7, 128, 661))


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "fp32")])
def test_chdecay_range_edges(d, dtype):
    """Channels at 0.1 (with bf16 and d = 128 below the MFMA pass's 1/8, so
    that head takes the vector-ALU output pass), at 1, and in between, across
    segment cuts."""
    H = 2
    alpha = np.empty((H, d), np.float32)
    alpha[0] = np.linspace(0.1, 1.0, d)
    alpha[1, : d // 2] = 0.1
    alpha[1, d // 2:] = 1.0
    run_ch_case(1, H, 1500, d, dtype, seed=635 + d, seg=512, alpha=alpha)


def test_chdecay_token_major():
    run_ch_case(2, 4, 700, 128, "bf16", seed=630, seg=256, token_major=True)


def test_chdecay_equal_channels_match_scalar_path():
    """All channels of a head at one decay: the channel-wise path agrees with
    the scalar-decay path (both within the bar of the oracle)."""
    torch = torch_mod()
    H, d = 4, 128
    lam = inputs.decay_schedule(H)
    alpha = np.repeat(lam[:, None], d, axis=1).astype(np.float32)
    out, fin = run_ch_case(1, H, 2048, d, "bf16", seed=640, seg=512, alpha=alpha)
    tq, tk, tv = inputs.device_qkv((1, H, 2048, d), 640, "bf16")
    out2, fin2 = la.lightning_attn_fwd(tq, tk, tv, torch.from_numpy(lam).cuda(), init_state=None)
    # (different initial states: compare only the scalar path against its oracle)
    q, k, v = (host(t) for t in (tq, tk, tv))
    o_ref, _, _ = oracle.fwd(q, k, v, lam)
    assert rel_err(host(out2), o_ref) <= TOL["bf16"]


def test_chdecay_full_layer_h64_n32k():
    """B=1 H=64 N=32768 d=128 bf16 with channel-wise decays, in the launch
    configuration the benchmark times: every output element and final-state
    entry of all 64 heads against the oracle's channel-wise recurrence."""
    torch = torch_mod()
    w = inputs.WORKLOADS["layer_h64_n32k"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    say("case full chdecay layer_h64_n32k")
    tq, tk, tv = inputs.device_qkv((B, H, N, d), w["seed"], "bf16")
    alpha = inputs.chdecay_schedule(H, d)
    out, fin = la.lightning_attn_fwd_chdecay(tq, tk, tv, torch.from_numpy(alpha).cuda(),
                                             block=w["block"])
    torch.cuda.synchronize()
    ORACLE_CACHE.clear()
    o_ref, f_ref = oracle.fwd_chdecay(host(tq), host(tk), host(tv), alpha)
    del tq, tk, tv
    eo = whole_rel_err(out, o_ref, dim=1, name="out")
    ef = whole_rel_err(fin, f_ref, dim=1, name="final_state")
    say("   err out %.3e state %.3e (all %d heads)" % (eo, ef, H))
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "bf16"), (128, "fp32"), (64, "fp32")])
def test_chdecay_decode_steps(d, dtype):
    """Channel-wise decode steps (state row i decays by alpha_i) against the
    oracle's channel-wise recurrence run one token at a time from the state."""
    torch = torch_mod()
    B, H, steps = 3, 4, 10
    say("case chdecay decode B=%d H=%d d=%d %s" % (B, H, d, dtype))
    q, k, v = inputs.host_qkv((steps, B, H, d), 650 + d, dtype=dtype)
    alpha = inputs.chdecay_schedule(H, d, 651)
    S0 = inputs.host_state((B, H, d, d), 652)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tq, tk, tv = (torch.from_numpy(x).cuda().to(tdt) for x in (q, k, v))
    st = torch.from_numpy(S0).cuda()
    ta = torch.from_numpy(alpha).cuda()
    S = S0.astype(np.float64)
    worst = 0.0
    for t in range(steps):
        o = la.lightning_attn_decode_chdecay(tq[t], tk[t], tv[t], ta, st)
        o_ref, S = oracle.fwd_chdecay(q[t][:, :, None], k[t][:, :, None], v[t][:, :, None], alpha,
                                      init=S)
        worst = max(worst, rel_err(host(o), o_ref[:, :, 0]))
    torch.cuda.synchronize()
    es = rel_err(host(st), S)
    say("   err out %.3e state %.3e" % (worst, es))
    assert worst <= TOL[dtype] and es <= TOL[dtype]


def test_chdecay_decode_continues_prefill():
    """Decoding token N-1 from the channel-wise prefill's state after N-1
    tokens reproduces the prefill's row N-1 (recurrent form)."""
    torch = torch_mod()
    B, H, N, d = 2, 4, 300, 128
    tq, tk, tv = inputs.device_qkv((B, H, N, d), 660, "bf16")
    ta = torch.from_numpy(inputs.chdecay_schedule(H, d, 661)).cuda()
    out, _ = la.lightning_attn_fwd_chdecay(tq, tk, tv, ta, segment_tokens=128)
    _, st = la.lightning_attn_fwd_chdecay(tq[:, :, :N - 1].contiguous(),
                                          tk[:, :, :N - 1].contiguous(),
                                          tv[:, :, :N - 1].contiguous(), ta, segment_tokens=128)
    o = la.lightning_attn_decode_chdecay(tq[:, :, N - 1].contiguous(),
                                         tk[:, :, N - 1].contiguous(),
                                         tv[:, :, N - 1].contiguous(), ta, st)
    torch.cuda.synchronize()
    e = rel_err(host(o), host(out[:, :, N - 1]))
    say("   decode vs prefill row: %.3e" % e)
    assert e <= TOL["bf16"]


def test_chdecay_empty_sequences_keep_the_state():
    torch = torch_mod()
    B, H, d = 2, 3, 128
    q = torch.empty(B, H, 0, d, dtype=torch.bfloat16, device="cuda")
    init = torch.randn(B, H, d, d, device="cuda")
    ta = torch.from_numpy(inputs.chdecay_schedule(H, d)).cuda()
    _, fin = la.lightning_attn_fwd_chdecay(q, q.clone(), q.clone(), ta, init_state=init)
    torch.cuda.synchronize()
    assert torch.equal(fin, init)


def run_ch_varlen_case(lens, H, d, dtype, seed, seg=0, with_init=True, token_major=False,
                       alpha=None):
    """Packed channel-wise prefill against the oracle's channel-wise
    recurrence run on each sequence on its own."""
    torch = torch_mod()
    say("case chdecay varlen lens=%s H=%d d=%d %s seg=%d init=%s token_major=%s"
        % (lens[:8], H, d, dtype, seg, with_init, token_major))
    cu = inputs.cu_seqlens(lens)
    total, S = int(cu[-1]), len(lens)
    q, k, v = inputs.host_qkv((H, total, d), seed, dtype=dtype)
    alpha = inputs.chdecay_schedule(H, d, seed + 1) if alpha is None else alpha
    init = inputs.host_state((S, H, d, d), seed + 2) if with_init else None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tq, tk, tv = (torch.from_numpy(x).cuda().to(tdt) for x in (q, k, v))
    layout = la.LA_HEAD_MAJOR
    if token_major:
        tq, tk, tv = (t.transpose(0, 1).contiguous() for t in (tq, tk, tv))
        layout = la.LA_TOKEN_MAJOR
    out = torch.full_like(tq, float("nan"))
    out, fins = la.lightning_attn_fwd_chdecay_varlen(
        tq, tk, tv, torch.from_numpy(alpha).cuda(), torch.from_numpy(cu).cuda(), layout=layout,
        init_states=None if init is None else torch.from_numpy(init).cuda(), segment_tokens=seg,
        out=out)
    torch.cuda.synchronize()
    if token_major:
        out = out.transpose(0, 1)
    ho, hf = host(out), host(fins)
    assert np.isfinite(ho).all()
    o_ref = np.zeros((H, total, d))
    f_ref = np.zeros((S, H, d, d))
    for j in range(S):
        a, b = int(cu[j]), int(cu[j + 1])
        oj, fj = oracle.fwd_chdecay(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], alpha,
                                    init=None if init is None else init[j][None])
        o_ref[:, a:b] = oj[0]
        f_ref[j] = fj[0]
    eo, ef = rel_err(ho, o_ref), rel_err(hf, f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL[dtype] and ef <= TOL[dtype], (eo, ef)


@pytest.mark.parametrize("seg", [0, 64, 200, 1000])
def test_chdecay_varlen(seg):
    """Packed sequences with empty ones among them, under segment cuts that
    fall inside sequences and inside 64-token chunks."""
    run_ch_varlen_case([300, 0, 1000, 7, 0, 2000, 129], 4, 128, "bf16", seed=700, seg=seg)


@pytest.mark.parametrize("d,dtype,token_major,with_init", [(128, "bf16", True, False),
                                                           (64, "fp32", False, True),
                                                           (128, "fp32", True, True)])
def test_chdecay_varlen_layouts_and_vector_alu(d, dtype, token_major, with_init):
    run_ch_varlen_case([500, 1, 700, 64], 3, d, dtype, seed=701, seg=128,
                       token_major=token_major, with_init=with_init)


def test_chdecay_varlen_rejects_one_segment_per_sequence():
    torch = torch_mod()
    H, d = 2, 128
    q = torch.zeros(H, 10, d, dtype=torch.bfloat16, device="cuda")
    alpha = torch.full((H, d), 0.9, device="cuda")
    cu = torch.tensor([0, 4, 10], dtype=torch.int32, device="cuda")
    with pytest.raises(la.LightningAttnError, match="LA_ERR_UNSUPPORTED"):
        la.lightning_attn_fwd_chdecay_varlen(q, q.clone(), q.clone(), alpha, cu,
                                             segment_tokens=la.LA_SEGMENT_PER_SEQUENCE)
