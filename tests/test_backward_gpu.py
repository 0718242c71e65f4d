"""GPU parity of the backward pass (lightning_attn_bwd) against the CPU
oracle's hand-derived gradient of the recurrence (oracle.bwd, pinned to the
matrix-form gradient and to finite differences).

Bar as for the forward pass: max |x - x_ref| / max |x_ref| <= 1e-4 for
float32 inputs, <= 2e-2 for bf16 inputs, for each of dq, dk, dv and the
initial-state gradient.
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


def run_bwd_case(B, H, N, d, dtype, seed, block=128, seg=0, with_init=True, with_dfin=True,
                 lam=None, token_major=False, saved=False):
    """saved: the training pair -- lightning_attn_fwd_save (its out and final
    state checked against the oracle's forward), then lightning_attn_bwd_saved,
    whose dk, dv and dinit must also equal lightning_attn_bwd's bit for bit
    (same kernels on the same inputs; only dq takes the saved states)."""
    torch = torch_mod()
    say("case bwd B=%d H=%d N=%d d=%d %s seg=%d init=%s dfin=%s token_major=%s saved=%s"
        % (B, H, N, d, dtype, seg, with_init, with_dfin, token_major, saved))
    q, k, v = inputs.host_qkv((B, H, N, d), seed, dtype=dtype)
    do, _, _ = inputs.host_qkv((B, H, N, d), seed + 1, dtype=dtype)
    lam = inputs.decay_schedule(H) if lam is None else np.asarray(lam, np.float32)
    init = inputs.host_state((B, H, d, d), seed + 2) if with_init else None
    dfin = inputs.host_state((B, H, d, d), seed + 3) if with_dfin else None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tq, tk, tv, tdo = (torch.from_numpy(x).cuda().to(tdt) for x in (q, k, v, do))
    layout = la.LA_HEAD_MAJOR
    if token_major:
        tq, tk, tv, tdo = (t.transpose(1, 2).contiguous() for t in (tq, tk, tv, tdo))
        layout = la.LA_TOKEN_MAJOR
    outs = [torch.full_like(tq, float("nan")) for _ in range(3)]
    tl = torch.from_numpy(lam).cuda()
    td = None if dfin is None else torch.from_numpy(dfin).cuda()
    ti = None if init is None else torch.from_numpy(init).cuda()
    if saved:
        out, fin, sv = la.lightning_attn_fwd_save(tq, tk, tv, tl, layout=layout, block=block,
                                                  init_state=ti, segment_tokens=seg)
        nsv = la.lightning_attn_saved_states_size(B, H, N, d, block, la._dtype_code(tq), seg)
        assert (sv is None) == (nsv == 0)
        dq, dk, dv, dinit = la.lightning_attn_bwd_saved(
            tq, tk, tv, tl, tdo, sv, dfinal=td, init_state=ti, layout=layout, block=block,
            segment_tokens=seg, dq=outs[0], dk=outs[1], dv=outs[2])
        _, pk, pv, pinit = la.lightning_attn_bwd(tq, tk, tv, tl, tdo, dfinal=td, init_state=ti,
                                                 layout=layout, block=block, segment_tokens=seg)
        torch.cuda.synchronize()
        assert torch.equal(dk, pk) and torch.equal(dv, pv) and torch.equal(dinit, pinit)
        if token_major:
            out = out.transpose(1, 2)
        o_ref, f_ref, _ = oracle.fwd(q, k, v, lam, init=init)
        eo, ef = rel_err(host(out), o_ref), rel_err(host(fin), f_ref)
        say("   saved %d bytes; forward err out %.3e state %.3e" % (nsv, eo, ef))
        assert eo <= TOL[dtype] and ef <= TOL[dtype], (eo, ef)
    else:
        dq, dk, dv, dinit = la.lightning_attn_bwd(
            tq, tk, tv, tl, tdo, dfinal=td, init_state=ti, layout=layout, block=block,
            segment_tokens=seg, dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.synchronize()
    if token_major:
        dq, dk, dv = (t.transpose(1, 2) for t in (dq, dk, dv))
    ref = oracle.bwd(q, k, v, lam, do, dfin=dfin, init=init)
    errs = []
    for name, got, want in zip(("dq", "dk", "dv", "dinit"), (dq, dk, dv, dinit), ref):
        g = host(got)
        assert np.isfinite(g).all(), name + " has unwritten or non-finite elements"
        errs.append(rel_err(g, want))
    say("   err dq %.3e dk %.3e dv %.3e dinit %.3e" % tuple(errs))
    assert max(errs) <= TOL[dtype], errs


def test_bwd_tiny_fp32():
    run_bwd_case(1, 2, 256, 64, "fp32", seed=500, block=64)


def test_bwd_mid_bf16():
    run_bwd_case(2, 8, 4096, 128, "bf16", seed=501, block=64)


@pytest.mark.parametrize("seg", [4096, 128, 640, 1000, la.LA_SEGMENT_PER_SEQUENCE])
def test_bwd_segment_split_invariance(seg):
    """The causal and the two time-reversed passes under every segment cut:
    reversed segments start inside sequences and hand states backwards."""
    run_bwd_case(2, 4, 4096, 128, "bf16", seed=502, seg=seg)


@pytest.mark.parametrize("N", [1, 2, 127, 128, 129, 300, 1000])
def test_bwd_ragged_tails(N):
    run_bwd_case(2, 3, N, 128, "bf16", seed=510 + N, lam=[0.9961, 0.3997, 0.75])


@pytest.mark.parametrize("with_init,with_dfin", [(False, False), (True, False), (False, True)])
def test_bwd_optional_states(with_init, with_dfin):
    run_bwd_case(1, 4, 1500, 128, "bf16", seed=520, with_init=with_init, with_dfin=with_dfin,
                 seg=512)


@pytest.mark.parametrize("d,dtype", [(64, "fp32"), (128, "fp32"), (64, "bf16")])
@pytest.mark.parametrize("seg", [0, 64])
def test_bwd_vector_alu(d, dtype, seg):
    run_bwd_case(1, 3, 300, d, dtype, seed=530 + d, seg=seg, lam=[0.999, 0.5, 0.9])


@pytest.mark.parametrize("d,dtype,seg", [(128, "bf16", 0), (128, "bf16", 256), (64, "fp32", 0)])
def test_bwd_token_major(d, dtype, seg):
    run_bwd_case(2, 5, 1000, d, dtype, seed=540 + d, seg=seg, token_major=True)


@pytest.mark.parametrize("seg", [0, 128, 1000, la.LA_SEGMENT_PER_SEQUENCE])
def test_bwd_saved_states(seg):
    """The training pair under segment cuts (one segment per sequence keeps
    nothing: saved is None)."""
    run_bwd_case(2, 4, 4096, 128, "bf16", seed=560, seg=seg, saved=True)


@pytest.mark.parametrize("with_init,with_dfin", [(False, False), (True, True)])
def test_bwd_saved_optional_states(with_init, with_dfin):
    run_bwd_case(1, 4, 1500, 128, "bf16", seed=561, with_init=with_init, with_dfin=with_dfin,
                 seg=512, saved=True)


@pytest.mark.parametrize("d,dtype,seg,token_major", [(64, "fp32", 64, False),
                                                     (128, "fp32", 64, False),
                                                     (64, "bf16", 64, True),
                                                     (128, "bf16", 256, True)])
def test_bwd_saved_layouts_and_vector_alu(d, dtype, seg, token_major):
    run_bwd_case(2, 3, 700, d, dtype, seed=562 + d, seg=seg, lam=[0.999, 0.5, 0.9],
                 token_major=token_major, saved=True)


def test_bwd_empty_sequences():
    """N = 0: the initial-state gradient is dfinal."""
    torch = torch_mod()
    B, H, d = 2, 3, 128
    q = torch.empty(B, H, 0, d, dtype=torch.bfloat16, device="cuda")
    dfin = torch.randn(B, H, d, d, device="cuda")
    lam = torch.from_numpy(inputs.decay_schedule(H)).cuda()
    _, _, _, dinit = la.lightning_attn_bwd(q, q.clone(), q.clone(), lam, q.clone(), dfinal=dfin)
    torch.cuda.synchronize()
    assert torch.equal(dinit, dfin)


@pytest.mark.parametrize("saved", [False, True])
def test_bwd_full_layer_h64_n32k(saved):
    """B=1 H=64 N=32768 d=128 (the prefill headline shape), in the launch
    configuration the benchmark times (saved: through lightning_attn_fwd_save
    and lightning_attn_bwd_saved): every element of dq, dk, dv and dinit of
    all 64 heads against the oracle's backward."""
    torch = torch_mod()
    w = inputs.WORKLOADS["layer_h64_n32k"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    say("case full bwd layer_h64_n32k saved=%s" % saved)
    tq, tk, tv = inputs.device_qkv((B, H, N, d), w["seed"], "bf16")
    tdo, _, _ = inputs.device_qkv((B, H, N, d), w["seed"] + 7, "bf16")
    lam = inputs.decay_schedule(H)
    tl = torch.from_numpy(lam).cuda()
    if saved:
        _, _, sv = la.lightning_attn_fwd_save(tq, tk, tv, tl, block=w["block"])
        dq, dk, dv, dinit = la.lightning_attn_bwd_saved(tq, tk, tv, tl, tdo, sv, block=w["block"])
    else:
        dq, dk, dv, dinit = la.lightning_attn_bwd(tq, tk, tv, tl, tdo, block=w["block"])
    torch.cuda.synchronize()

    def compute():
        return oracle.bwd(host(tq), host(tk), host(tv), lam, host(tdo))

    ref = ORACLE_CACHE.get("bwd_layer_h64_n32k", compute)
    del tq, tk, tv, tdo
    errs = [whole_rel_err(g, r, dim=1, name=n)
            for n, g, r in zip(("dq", "dk", "dv", "dinit"), (dq, dk, dv, dinit), ref)]
    say("   err dq %.3e dk %.3e dv %.3e dinit %.3e (all %d heads)" % (tuple(errs) + (H,)))
    assert max(errs) <= TOL["bf16"], errs


@pytest.mark.parametrize("seg", [1024, la.LA_SEGMENT_PER_SEQUENCE])
def test_bwd_slow_decay(seg):
    """Heads with lambda <= 2^-15 (the kernels' per-power branch) beside
    ordinary heads: the anti-causal passes start from dfinal / lambda (1e19 at
    lambda = 1e-20, still finite in float32) and decay it at once."""
    run_bwd_case(1, 6, 3000, 128, "bf16", seed=540, seg=seg,
                 lam=[0.9, 2.0 ** -16, 1e-6, 1e-20, 0.5, 0.999])


def run_bwd_varlen_case(lens, H, d, dtype, seed, seg=0, with_states=True, token_major=False,
                        saved=False):
    """Packed backward against the oracle's backward run on each sequence
    (saved: through the packed training pair, as in run_bwd_case)."""
    torch = torch_mod()
    say("case bwd varlen lens=%s H=%d d=%d %s seg=%d states=%s token_major=%s saved=%s"
        % (lens[:8], H, d, dtype, seg, with_states, token_major, saved))
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    q, k, v = inputs.host_qkv((H, total, d), seed, dtype=dtype)
    do, _, _ = inputs.host_qkv((H, total, d), seed + 1, dtype=dtype)
    lam = inputs.decay_schedule(H)
    S = len(lens)
    init = inputs.host_state((S, H, d, d), seed + 2) if with_states else None
    dfin = inputs.host_state((S, H, d, d), seed + 3) if with_states else None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tq, tk, tv, tdo = (torch.from_numpy(x).cuda().to(tdt) for x in (q, k, v, do))
    layout = la.LA_HEAD_MAJOR
    if token_major:
        tq, tk, tv, tdo = (t.transpose(0, 1).contiguous() for t in (tq, tk, tv, tdo))
        layout = la.LA_TOKEN_MAJOR
    outs = [torch.full_like(tq, float("nan")) for _ in range(3)]
    tl, tcu = torch.from_numpy(lam).cuda(), torch.from_numpy(cu).cuda()
    td = None if dfin is None else torch.from_numpy(dfin).cuda()
    ti = None if init is None else torch.from_numpy(init).cuda()
    if saved:
        out, fins, sv = la.lightning_attn_fwd_varlen_save(tq, tk, tv, tl, tcu, layout=layout,
                                                          init_states=ti, segment_tokens=seg)
        nsv = la.lightning_attn_varlen_saved_states_size(S, H, total, d, 128, la._dtype_code(tq),
                                                         seg)
        assert (sv is None) == (nsv == 0)
        dq, dk, dv, dinit = la.lightning_attn_bwd_varlen_saved(
            tq, tk, tv, tl, tdo, tcu, sv, layout=layout, dfinals=td, init_states=ti,
            segment_tokens=seg, dq=outs[0], dk=outs[1], dv=outs[2])
        _, pk, pv, pinit = la.lightning_attn_bwd_varlen(tq, tk, tv, tl, tdo, tcu, layout=layout,
                                                        dfinals=td, init_states=ti,
                                                        segment_tokens=seg)
        torch.cuda.synchronize()
        assert torch.equal(dk, pk) and torch.equal(dv, pv) and torch.equal(dinit, pinit)
        if token_major:
            out = out.transpose(0, 1)
        o_ref, f_ref, _ = oracle.fwd_varlen(q, k, v, lam, cu, init=init)
        eo, ef = rel_err(host(out), o_ref), rel_err(host(fins), f_ref)
        say("   saved %d bytes; forward err out %.3e state %.3e" % (nsv, eo, ef))
        assert eo <= TOL[dtype] and ef <= TOL[dtype], (eo, ef)
    else:
        dq, dk, dv, dinit = la.lightning_attn_bwd_varlen(
            tq, tk, tv, tl, tdo, tcu, layout=layout, dfinals=td, init_states=ti,
            segment_tokens=seg, dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.synchronize()
    if token_major:
        dq, dk, dv = (t.transpose(0, 1) for t in (dq, dk, dv))
    hq, hk, hv, hi = (host(t) for t in (dq, dk, dv, dinit))
    refs = [np.zeros((H, total, d)) for _ in range(3)] + [np.zeros((S, H, d, d))]
    for j in range(S):
        a, b = int(cu[j]), int(cu[j + 1])
        r = oracle.bwd(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], lam, do[None, :, a:b],
                       dfin=None if dfin is None else dfin[j][None],
                       init=None if init is None else init[j][None])
        for t in range(3):
            refs[t][:, a:b] = r[t][0]
        refs[3][j] = r[3][0]
    errs = [rel_err(g, ref) for g, ref in zip((hq, hk, hv, hi), refs)]
    assert all(np.isfinite(x).all() for x in (hq, hk, hv, hi))
    say("   err dq %.3e dk %.3e dv %.3e dinit %.3e" % tuple(errs))
    assert max(errs) <= TOL[dtype], errs


@pytest.mark.parametrize("seg", [0, 200, 1000, la.LA_SEGMENT_PER_SEQUENCE])
def test_bwd_varlen(seg):
    """Packed sequences (empty ones first, inside and last; segments that cut
    sequences and hand states across the cut in both directions)."""
    run_bwd_varlen_case([0, 300, 0, 1, 129, 1024, 5, 640, 0], 4, 128, "bf16", seed=550 + seg,
                        seg=seg)


def test_bwd_varlen_token_major_no_states():
    run_bwd_varlen_case([300, 1, 129, 1024, 5], 4, 128, "bf16", seed=560, seg=256,
                        with_states=False, token_major=True)


@pytest.mark.parametrize("d,dtype", [(64, "fp32"), (128, "fp32"), (64, "bf16")])
def test_bwd_varlen_vector_alu(d, dtype):
    run_bwd_varlen_case([33, 0, 64, 1, 100], 2, d, dtype, seed=570 + d, seg=48)


@pytest.mark.parametrize("seg", [0, 200, la.LA_SEGMENT_PER_SEQUENCE])
def test_bwd_varlen_saved_states(seg):
    """The packed training pair, with empty sequences among the packed ones."""
    run_bwd_varlen_case([300, 0, 1000, 7, 0, 2000, 129], 4, 128, "bf16", seed=620, seg=seg,
                        saved=True)


@pytest.mark.parametrize("d,dtype,token_major", [(128, "bf16", True), (64, "fp32", False)])
def test_bwd_varlen_saved_layouts(d, dtype, token_major):
    run_bwd_varlen_case([500, 1, 700], 3, d, dtype, seed=621, seg=128, token_major=token_major,
                        saved=True)


def test_bwd_saved_states_are_what_dq_uses():
    """The dq pass of lightning_attn_bwd_saved really starts its segments
    from `saved`: with the forward's states zeroed, dq changes in every
    segment but the first (whose entering state is the initial state's, also
    zeroed here, which is the case where it is zero anyway) and stays put in
    the first; dk and dv do not depend on it."""
    torch = torch_mod()
    B, H, N, d, seg = 1, 2, 1024, 128, 256
    say("case bwd saved states are used")
    q, k, v = inputs.device_qkv((B, H, N, d), 640, "bf16")
    do, _, _ = inputs.device_qkv((B, H, N, d), 641, "bf16")
    lam = torch.tensor([0.999, 0.99], dtype=torch.float32, device="cuda")
    _, _, sv = la.lightning_attn_fwd_save(q, k, v, lam, segment_tokens=seg)
    dq, dk, dv, _ = la.lightning_attn_bwd_saved(q, k, v, lam, do, sv, segment_tokens=seg)
    zq, zk, zv, _ = la.lightning_attn_bwd_saved(q, k, v, lam, do, torch.zeros_like(sv),
                                                segment_tokens=seg)
    torch.cuda.synchronize()
    assert torch.equal(dk, zk) and torch.equal(dv, zv)
    assert torch.equal(dq[:, :, :seg], zq[:, :, :seg])
    for s in range(1, N // seg):
        part = slice(s * seg, (s + 1) * seg)
        assert not torch.equal(dq[:, :, part], zq[:, :, part]), s


def test_training_pair_graph_replay():
    """lightning_attn_fwd_save followed by lightning_attn_bwd_saved, captured
    as one HIP graph (a training step's attention), gives the eager results
    bit for bit on every replay, with eager work and synchronisations between
    the replays."""
    torch = torch_mod()
    B, H, N, d, seg = 1, 4, 2048, 128, 512
    say("case training pair graph replay")
    q, k, v = inputs.device_qkv((B, H, N, d), 650, "bf16")
    do, _, _ = inputs.device_qkv((B, H, N, d), 651, "bf16")
    lam = torch.from_numpy(inputs.decay_schedule(H)).cuda()
    init = inputs.device_state((B, H, d, d), 652)
    dfin = inputs.device_state((B, H, d, d), 653)
    out, fin = torch.empty_like(q), torch.empty_like(init)
    dq, dk, dv, dinit = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q),
                         torch.empty_like(init))
    nsv = la.lightning_attn_saved_states_size(B, H, N, d, 128, la.LA_BF16, seg)
    sv = torch.empty(nsv // 4, dtype=torch.float32, device="cuda")
    ws = torch.empty(la.lightning_attn_bwd_workspace_size(B, H, N, d, 128, la.LA_BF16, seg),
                     dtype=torch.uint8, device="cuda")

    def step():
        la.lightning_attn_fwd_save(q, k, v, lam, init_state=init, segment_tokens=seg, out=out,
                                   final_state=fin, saved=sv, workspace=ws)
        la.lightning_attn_bwd_saved(q, k, v, lam, do, sv, dfinal=dfin, init_state=init,
                                    segment_tokens=seg, dq=dq, dk=dk, dv=dv, dinit=dinit,
                                    workspace=ws)

    step()
    torch.cuda.synchronize()
    outs = (out, fin, sv, dq, dk, dv, dinit)
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("out", "final", "saved", "dq", "dk", "dv", "dinit"), outs,
                                   ref):
            assert torch.equal(got, want), "replay %d: %s differs" % (r, name)
