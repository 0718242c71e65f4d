"""GPU parity over a seeded random sweep of configurations.

Each case draws its shape, dtype, block, segment length, layout, initial
state and decays from a fixed seed, runs the HIP path through the C ABI and
compares every output and state element with the double-precision oracle
(max |x - x_ref| / max |x_ref| <= 1e-4 for float32 inputs, 2e-2 for bf16).
The draws mix sizes around the chunk lengths (1 token, a ragged tail,
several segments), decays from the schedule, close to 1 and very small,
empty packed sequences, and every entry-point family: fixed-length and
packed prefill, the gated reading, the channel-wise variant and the
backward pass.  The case index is printed first, so a failure names it.
"""
import sys

import numpy as np
import pytest

import oracle
import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}
BLOCKS = [16, 32, 64, 128, 256]


def torch_mod():
    import torch
    return torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert np.isfinite(a).all()
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0))


def host(t):
    torch = torch_mod()
    return t.detach().to(torch.float32).cpu().numpy()


def dev(x, dtype):
    torch = torch_mod()
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(tdt)


def draw_decays(g, H):
    """Per-head decays: the schedule, values close to 1, or small ones (the
    factored-power and per-power branches of the kernels alike)."""
    kind = g.integers(0, 3)
    if kind == 0:
        return inputs.decay_schedule(H)
    if kind == 1:
        return (1.0 - 10.0 ** g.uniform(-4, -1, H)).astype(np.float32)
    return np.exp2(-g.uniform(0.05, 24, H)).astype(np.float32)


def draw_common(g):
    d = int(g.choice([64, 128]))
    dtype = str(g.choice(["bf16", "fp32"]))
    block = int(g.choice(BLOCKS))
    return d, dtype, block


def draw_seg(g, n):
    """Automatic, one segment per sequence, or a random cut (possibly not a
    multiple of any chunk)."""
    kind = g.integers(0, 4)
    if kind == 0:
        return 0
    if kind == 1:
        return la.LA_SEGMENT_PER_SEQUENCE
    return int(g.integers(1, max(2, n)))


def draw_n(g):
    kind = g.integers(0, 4)
    if kind == 0:
        return int(g.integers(1, 4))
    if kind == 1:
        return int(g.choice([64, 128, 256])) + int(g.integers(-1, 2))
    return int(g.integers(1, 1400))


FIXED_CASES = 24


@pytest.mark.parametrize("case", range(FIXED_CASES))
def test_random_fixed(case):
    g = np.random.default_rng(9000 + case)
    B, H = int(g.integers(1, 4)), int(g.integers(1, 6))
    N = draw_n(g)
    d, dtype, block = draw_common(g)
    seg = draw_seg(g, N)
    token_major = bool(g.integers(0, 2))
    with_init = bool(g.integers(0, 2))
    lam = draw_decays(g, H)
    say("case fixed %d: B=%d H=%d N=%d d=%d %s block=%d seg=%d token_major=%s init=%s lam=%s"
        % (case, B, H, N, d, dtype, block, seg, token_major, with_init,
           np.array2string(lam, precision=3)))
    q, k, v = inputs.host_qkv((B, H, N, d), 9100 + case, dtype=dtype)
    init = inputs.host_state((B, H, d, d), 9200 + case) if with_init else None
    tq, tk, tv = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    layout = la.LA_HEAD_MAJOR
    if token_major:
        tq, tk, tv = (t.transpose(1, 2).contiguous() for t in (tq, tk, tv))
        layout = la.LA_TOKEN_MAJOR
    out, fin = la.lightning_attn_fwd_layout(
        tq, tk, tv, dev(lam, "fp32"), layout, block=block,
        init_state=None if init is None else dev(init, "fp32"), segment_tokens=seg)
    torch_mod().cuda.synchronize()
    if token_major:
        out = out.transpose(1, 2)
    o_ref, f_ref, _ = oracle.fwd(q, k, v, lam, init=init)
    eo, ef = rel_err(host(out), o_ref), rel_err(host(fin), f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


VARLEN_CASES = 16


@pytest.mark.parametrize("case", range(VARLEN_CASES))
def test_random_varlen(case):
    g = np.random.default_rng(9300 + case)
    S, H = int(g.integers(1, 9)), int(g.integers(1, 5))
    lens = [0 if g.random() < 0.2 else draw_n(g) for _ in range(S)]
    if sum(lens) == 0:
        lens[-1] = 1
    total = int(sum(lens))
    d, dtype, block = draw_common(g)
    seg = draw_seg(g, max(total, 1))
    with_init = bool(g.integers(0, 2))
    lam = draw_decays(g, H)
    say("case varlen %d: lens=%s H=%d d=%d %s block=%d seg=%d init=%s"
        % (case, lens, H, d, dtype, block, seg, with_init))
    cu = inputs.cu_seqlens(lens)
    q, k, v = inputs.host_qkv((H, total, d), 9400 + case, dtype=dtype)
    init = inputs.host_state((S, H, d, d), 9500 + case) if with_init else None
    torch = torch_mod()
    out, fin = la.lightning_attn_fwd_varlen(
        dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(lam, "fp32"),
        torch.from_numpy(cu).to("cuda"), block=block,
        init_states=None if init is None else dev(init, "fp32"), segment_tokens=seg)
    torch.cuda.synchronize()
    o_ref, f_ref, _ = oracle.fwd_varlen(q, k, v, lam, cu, init=init)
    eo, ef = rel_err(host(out), o_ref), rel_err(host(fin), f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


GATED_CASES = 8


@pytest.mark.parametrize("case", range(GATED_CASES))
def test_random_gated(case):
    g = np.random.default_rng(9600 + case)
    B, H = int(g.integers(1, 3)), int(g.integers(1, 5))
    N = draw_n(g)
    d = 128
    flags = int(g.integers(1, 32))
    seg = draw_seg(g, N)
    lam = draw_decays(g, H)
    say("case gated %d: B=%d H=%d N=%d flags=%d seg=%d" % (case, B, H, N, flags, seg))
    q, k, v = inputs.host_qkv((B, H, N, d), 9700 + case, dtype="bf16")
    gate, _, _ = inputs.host_qkv((B, H, N, d), 9701 + case, dtype="bf16")
    gate = inputs.round_to_bf16(gate * np.float32(2.0 * np.sqrt(d)))
    wgt = g.uniform(0.5, 1.5, (H, d)).astype(np.float32)
    out, fin = la.lightning_attn_fwd_gated(
        dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(lam, "fp32"), flags,
        gate=dev(gate, "bf16"), norm_weight=dev(wgt, "fp32"), eps=1e-5, segment_tokens=seg)
    torch_mod().cuda.synchronize()
    o_ref, f_ref = oracle.fwd_gated(q, k, v, lam, flags, gate=gate, weight=wgt, eps=1e-5)
    eo, ef = rel_err(host(out), o_ref), rel_err(host(fin), f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


CH_CASES = 8


@pytest.mark.parametrize("case", range(CH_CASES))
def test_random_chdecay(case):
    g = np.random.default_rng(9800 + case)
    B, H = int(g.integers(1, 3)), int(g.integers(1, 5))
    N = draw_n(g)
    d, dtype, block = draw_common(g)
    seg = draw_seg(g, N)
    # per-channel decays: some heads entirely above 1/8, some with channels
    # below it (those heads take the vector-ALU output pass)
    # (log2 of each channel's rate uniform in [-10, hi_h], hi_h per head in
    # [-3, 3]: a head whose hi_h is below log2(ln 8) has every alpha >= 1/8)
    hi = g.uniform(-3, 3, (H, 1))
    log2_rate = -10.0 + g.uniform(0, 1, (H, d)) * (hi + 10.0)
    alpha = np.exp(-np.exp2(log2_rate)).astype(np.float32)
    alpha[:, 0] = 1.0
    say("case chdecay %d: B=%d H=%d N=%d d=%d %s block=%d seg=%d min alpha %s"
        % (case, B, H, N, d, dtype, block, seg, np.array2string(alpha.min(1), precision=3)))
    q, k, v = inputs.host_qkv((B, H, N, d), 9900 + case, dtype=dtype)
    out, fin = la.lightning_attn_fwd_chdecay(dev(q, dtype), dev(k, dtype), dev(v, dtype),
                                             dev(alpha, "fp32"), block=block,
                                             segment_tokens=seg)
    torch_mod().cuda.synchronize()
    o_ref, f_ref = oracle.fwd_chdecay(q, k, v, alpha)
    eo, ef = rel_err(host(out), o_ref), rel_err(host(fin), f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


BWD_CASES = 8


@pytest.mark.parametrize("case", range(BWD_CASES))
def test_random_backward(case):
    g = np.random.default_rng(10000 + case)
    B, H = int(g.integers(1, 3)), int(g.integers(1, 4))
    N = draw_n(g)
    d, dtype, _ = draw_common(g)
    seg = draw_seg(g, N)
    token_major = bool(g.integers(0, 2))
    # the reversed passes start from dS_fin / lambda: keep lambda away from 0
    lam = np.exp2(-g.uniform(0.01, 6, H)).astype(np.float32)
    say("case bwd %d: B=%d H=%d N=%d d=%d %s seg=%d token_major=%s"
        % (case, B, H, N, d, dtype, seg, token_major))
    q, k, v = inputs.host_qkv((B, H, N, d), 10100 + case, dtype=dtype)
    do, _, _ = inputs.host_qkv((B, H, N, d), 10101 + case, dtype=dtype)
    dfin = inputs.host_state((B, H, d, d), 10102 + case)
    init = inputs.host_state((B, H, d, d), 10103 + case)
    tq, tk, tv, tdo = dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(do, dtype)
    layout = la.LA_HEAD_MAJOR
    if token_major:
        tq, tk, tv, tdo = (t.transpose(1, 2).contiguous() for t in (tq, tk, tv, tdo))
        layout = la.LA_TOKEN_MAJOR
    dq, dk, dv, dinit = la.lightning_attn_bwd(tq, tk, tv, dev(lam, "fp32"), tdo,
                                              dfinal=dev(dfin, "fp32"),
                                              init_state=dev(init, "fp32"), layout=layout,
                                              segment_tokens=seg)
    torch_mod().cuda.synchronize()
    if token_major:
        dq, dk, dv = (t.transpose(1, 2) for t in (dq, dk, dv))
    rq, rk, rv, ri = oracle.bwd(q, k, v, lam, do, dfin=dfin, init=init)
    errs = [rel_err(host(a), b) for a, b in ((dq, rq), (dk, rk), (dv, rv), (dinit, ri))]
    say("   err dq %.3e dk %.3e dv %.3e dinit %.3e" % tuple(errs))
    assert max(errs) <= TOL[dtype]
