"""GPU parity over a seeded random sweep of the entry points that the
fixed-length sweep leaves out: packed gated prefill, packed channel-wise
decay, the packed backward, both training pairs (forward with saved states,
then the backward that uses them), prefix-state snapshots, decode steps
(scalar and channel-wise), the allocation-free prefill, token-major packed
prefill and the mixed serving step.

Each case draws its shapes, lengths (empty sequences among them), dtype,
block, segment policy, initial states and decays from a fixed seed, runs the
HIP path through the C ABI and compares every output and state element with
the double-precision oracle (max |x - x_ref| / max |x_ref| <= 1e-4 for
float32 inputs, 2e-2 for bf16).  A packed sequence is compared with the
oracle's recurrence over that sequence alone (sequences are independent).
The case is printed before it runs, so a failure names it.
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
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.isfinite(a).all()
    if a.size == 0:
        return 0.0
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0))


def host(t):
    torch = torch_mod()
    return t.detach().to(torch.float32).cpu().numpy()


def dev(x, dtype):
    torch = torch_mod()
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(tdt)


def dev_i32(x):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda")


def sync():
    torch_mod().cuda.synchronize()


def draw_decays(g, H):
    kind = g.integers(0, 3)
    if kind == 0:
        return inputs.decay_schedule(H)
    if kind == 1:
        return (1.0 - 10.0 ** g.uniform(-4, -1, H)).astype(np.float32)
    return np.exp2(-g.uniform(0.05, 24, H)).astype(np.float32)


def draw_len(g):
    kind = g.integers(0, 5)
    if kind == 0:
        return 0
    if kind == 1:
        return int(g.integers(1, 4))
    if kind == 2:
        return int(g.choice([64, 128, 256])) + int(g.integers(-1, 2))
    return int(g.integers(1, 900))


def draw_lens(g, smax):
    S = int(g.integers(1, smax + 1))
    lens = [draw_len(g) for _ in range(S)]
    if sum(lens) == 0:
        lens[-1] = 1
    return lens


def draw_seg(g, n):
    kind = g.integers(0, 4)
    if kind == 0:
        return 0
    if kind == 1:
        return la.LA_SEGMENT_PER_SEQUENCE
    return int(g.integers(1, max(2, n)))


def draw_common(g, dtypes=("bf16", "fp32")):
    d = int(g.choice([64, 128]))
    dtype = str(g.choice(list(dtypes)))
    block = int(g.choice(BLOCKS))
    return d, dtype, block


def seq_slice(x, cu, j):
    """Sequence j of a packed head-major [H, total, d] array as [1, H, n, d]."""
    return x[None, :, cu[j]:cu[j + 1], :]


def to_token_major(t):
    # [H, total, d] -> [total, H, d]
    return t.transpose(0, 1).contiguous()


def oracle_packed(fn, cu, arrays, init=None, **kw):
    """Runs fn (an oracle function over [1, H, n, d] inputs returning (out,
    fin, ...)) over each sequence; returns (out [H, total, d], fins [S, H,
    d, d])."""
    S = len(cu) - 1
    H, total, d = arrays[0].shape
    out = np.zeros((H, total, d), np.float64)
    fins = np.zeros((S, H, d, d), np.float64)
    for j in range(S):
        ij = None if init is None else init[j:j + 1]
        if cu[j + 1] == cu[j]:
            fins[j] = 0.0 if init is None else init[j]
            continue
        res = fn(*[seq_slice(a, cu, j) for a in arrays], init=ij, **kw)
        out[:, cu[j]:cu[j + 1]] = res[0][0]
        fins[j] = res[1][0]
    return out, fins


# ---------------------------------------------------------------------------
# packed gated prefill

GATED_VARLEN_CASES = 8


@pytest.mark.parametrize("case", range(GATED_VARLEN_CASES))
def test_random_gated_varlen(case):
    g = np.random.default_rng(20000 + case)
    H = int(g.integers(1, 5))
    lens = draw_lens(g, 6)
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    d = 128
    flags = int(g.integers(0, 32))
    seg = draw_seg(g, total)
    token_major = bool(g.integers(0, 2))
    with_init = bool(g.integers(0, 2))
    lam = draw_decays(g, H)
    eps = float(g.choice([1e-6, 1e-5]))
    say("case gated varlen %d: lens=%s H=%d flags=%d seg=%d token_major=%s init=%s"
        % (case, lens, H, flags, seg, token_major, with_init))
    q, k, v = inputs.host_qkv((H, total, d), 20100 + case, dtype="bf16")
    gate, _, _ = inputs.host_qkv((H, total, d), 20101 + case, dtype="bf16")
    gate = inputs.round_to_bf16(gate * np.float32(2.0 * np.sqrt(d)))
    wgt = g.uniform(0.5, 1.5, (H, d)).astype(np.float32)
    S = len(lens)
    init = inputs.host_state((S, H, d, d), 20102 + case) if with_init else None
    tq, tk, tv, tg = (dev(x, "bf16") for x in (q, k, v, gate))
    layout = la.LA_HEAD_MAJOR
    if token_major:
        tq, tk, tv, tg = (to_token_major(t) for t in (tq, tk, tv, tg))
        layout = la.LA_TOKEN_MAJOR
    out, fin = la.lightning_attn_fwd_varlen_gated(
        tq, tk, tv, dev(lam, "fp32"), dev_i32(cu), flags, gate=tg, norm_weight=dev(wgt, "fp32"),
        eps=eps, layout=layout, init_states=None if init is None else dev(init, "fp32"),
        segment_tokens=seg)
    sync()
    if token_major:
        out = out.transpose(0, 1)

    def fn(qq, kk, vv, gg, init=None):
        return oracle.fwd_gated(qq, kk, vv, lam, flags, gate=gg, weight=wgt, eps=eps, init=init)

    o_ref, f_ref = oracle_packed(fn, cu, (q, k, v, gate), init=init)
    eo, ef = rel_err(host(out), o_ref), rel_err(host(fin), f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


# ---------------------------------------------------------------------------
# packed channel-wise decay

CH_VARLEN_CASES = 6


@pytest.mark.parametrize("case", range(CH_VARLEN_CASES))
def test_random_chdecay_varlen(case):
    g = np.random.default_rng(21000 + case)
    H = int(g.integers(1, 4))
    lens = draw_lens(g, 5)
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    d, dtype, block = draw_common(g)
    seg = draw_seg(g, total)
    token_major = bool(g.integers(0, 2))
    with_init = bool(g.integers(0, 2))
    # some heads with every alpha >= 1/8, some with channels below
    hi = g.uniform(-3, 3, (H, 1))
    alpha = np.exp(-np.exp2(-10.0 + g.uniform(0, 1, (H, d)) * (hi + 10.0))).astype(np.float32)
    say("case chdecay varlen %d: lens=%s H=%d d=%d %s block=%d seg=%d token_major=%s init=%s"
        % (case, lens, H, d, dtype, block, seg, token_major, with_init))
    q, k, v = inputs.host_qkv((H, total, d), 21100 + case, dtype=dtype)
    S = len(lens)
    init = inputs.host_state((S, H, d, d), 21101 + case) if with_init else None
    tq, tk, tv = (dev(x, dtype) for x in (q, k, v))
    layout = la.LA_HEAD_MAJOR
    if token_major:
        tq, tk, tv = (to_token_major(t) for t in (tq, tk, tv))
        layout = la.LA_TOKEN_MAJOR
    out, fin = la.lightning_attn_fwd_chdecay_varlen(
        tq, tk, tv, dev(alpha, "fp32"), dev_i32(cu), layout=layout, block=block,
        init_states=None if init is None else dev(init, "fp32"), segment_tokens=seg)
    sync()
    if token_major:
        out = out.transpose(0, 1)

    def fn(qq, kk, vv, init=None):
        return oracle.fwd_chdecay(qq, kk, vv, alpha, init=init)

    o_ref, f_ref = oracle_packed(fn, cu, (q, k, v), init=init)
    eo, ef = rel_err(host(out), o_ref), rel_err(host(fin), f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


# ---------------------------------------------------------------------------
# packed backward, and both training pairs


def bwd_lambdas(g, H):
    # the reversed passes start from dS_fin / lambda: keep lambda away from 0
    return np.exp2(-g.uniform(0.01, 6, H)).astype(np.float32)


def oracle_bwd_packed(cu, q, k, v, lam, do, dfin, init):
    S = len(cu) - 1
    H, total, d = q.shape
    grads = [np.zeros((H, total, d), np.float64) for _ in range(3)]
    dinit = np.zeros((S, H, d, d), np.float64)
    for j in range(S):
        if cu[j + 1] == cu[j]:
            dinit[j] = 0.0 if dfin is None else dfin[j]  # the state passes through unchanged
            continue
        sl = [seq_slice(a, cu, j) for a in (q, k, v)]
        r = oracle.bwd(*sl, lam, seq_slice(do, cu, j),
                       dfin=None if dfin is None else dfin[j:j + 1],
                       init=None if init is None else init[j:j + 1])
        for gr, x in zip(grads, r[:3]):
            gr[:, cu[j]:cu[j + 1]] = x[0]
        dinit[j] = r[3][0]
    return grads[0], grads[1], grads[2], dinit


BWD_VARLEN_CASES = 6


@pytest.mark.parametrize("case", range(BWD_VARLEN_CASES))
def test_random_backward_varlen(case):
    g = np.random.default_rng(22000 + case)
    H = int(g.integers(1, 4))
    lens = draw_lens(g, 5)
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    d, dtype, _ = draw_common(g)
    seg = draw_seg(g, total)
    token_major = bool(g.integers(0, 2))
    with_init, with_dfin = bool(g.integers(0, 2)), bool(g.integers(0, 2))
    lam = bwd_lambdas(g, H)
    S = len(lens)
    say("case bwd varlen %d: lens=%s H=%d d=%d %s seg=%d token_major=%s init=%s dfin=%s"
        % (case, lens, H, d, dtype, seg, token_major, with_init, with_dfin))
    q, k, v = inputs.host_qkv((H, total, d), 22100 + case, dtype=dtype)
    do, _, _ = inputs.host_qkv((H, total, d), 22101 + case, dtype=dtype)
    init = inputs.host_state((S, H, d, d), 22102 + case) if with_init else None
    dfin = inputs.host_state((S, H, d, d), 22103 + case) if with_dfin else None
    tq, tk, tv, tdo = (dev(x, dtype) for x in (q, k, v, do))
    layout = la.LA_HEAD_MAJOR
    if token_major:
        tq, tk, tv, tdo = (to_token_major(t) for t in (tq, tk, tv, tdo))
        layout = la.LA_TOKEN_MAJOR
    dq, dk, dv, dinit = la.lightning_attn_bwd_varlen(
        tq, tk, tv, dev(lam, "fp32"), tdo, dev_i32(cu), layout=layout,
        dfinals=None if dfin is None else dev(dfin, "fp32"),
        init_states=None if init is None else dev(init, "fp32"), segment_tokens=seg)
    sync()
    if token_major:
        dq, dk, dv = (t.transpose(0, 1) for t in (dq, dk, dv))
    ref = oracle_bwd_packed(cu, q, k, v, lam, do, dfin, init)
    errs = [rel_err(host(a), b) for a, b in zip((dq, dk, dv, dinit), ref)]
    say("   err dq %.3e dk %.3e dv %.3e dinit %.3e" % tuple(errs))
    assert max(errs) <= TOL[dtype]


PAIR_CASES = 5


@pytest.mark.parametrize("case", range(PAIR_CASES))
def test_random_training_pair(case):
    g = np.random.default_rng(23000 + case)
    B, H = int(g.integers(1, 3)), int(g.integers(1, 4))
    N = int(g.choice([1, 2, 127, 128, 129])) if g.integers(0, 2) else int(g.integers(1, 1200))
    d, dtype, block = draw_common(g)
    seg = draw_seg(g, N)
    token_major = bool(g.integers(0, 2))
    lam = bwd_lambdas(g, H)
    say("case pair %d: B=%d H=%d N=%d d=%d %s block=%d seg=%d token_major=%s"
        % (case, B, H, N, d, dtype, block, seg, token_major))
    q, k, v = inputs.host_qkv((B, H, N, d), 23100 + case, dtype=dtype)
    do, _, _ = inputs.host_qkv((B, H, N, d), 23101 + case, dtype=dtype)
    init = inputs.host_state((B, H, d, d), 23102 + case)
    dfin = inputs.host_state((B, H, d, d), 23103 + case)
    tq, tk, tv, tdo = (dev(x, dtype) for x in (q, k, v, do))
    layout = la.LA_HEAD_MAJOR
    if token_major:
        tq, tk, tv, tdo = (t.transpose(1, 2).contiguous() for t in (tq, tk, tv, tdo))
        layout = la.LA_TOKEN_MAJOR
    tl, ti = dev(lam, "fp32"), dev(init, "fp32")
    out, fin, saved = la.lightning_attn_fwd_save(tq, tk, tv, tl, layout=layout, block=block,
                                                 init_state=ti, segment_tokens=seg)
    dq, dk, dv, dinit = la.lightning_attn_bwd_saved(tq, tk, tv, tl, tdo, saved,
                                                    dfinal=dev(dfin, "fp32"), init_state=ti,
                                                    layout=layout, block=block,
                                                    segment_tokens=seg)
    sync()
    if token_major:
        out, dq, dk, dv = (t.transpose(1, 2) for t in (out, dq, dk, dv))
    o_ref, f_ref, _ = oracle.fwd(q, k, v, lam, init=init)
    ref = oracle.bwd(q, k, v, lam, do, dfin=dfin, init=init)
    errs = [rel_err(host(out), o_ref), rel_err(host(fin), f_ref)]
    errs += [rel_err(host(a), b) for a, b in zip((dq, dk, dv, dinit), ref)]
    say("   err out %.3e state %.3e dq %.3e dk %.3e dv %.3e dinit %.3e" % tuple(errs))
    assert max(errs) <= TOL[dtype]


PAIR_VARLEN_CASES = 4


@pytest.mark.parametrize("case", range(PAIR_VARLEN_CASES))
def test_random_training_pair_varlen(case):
    g = np.random.default_rng(24000 + case)
    H = int(g.integers(1, 4))
    lens = draw_lens(g, 5)
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    d, dtype, block = draw_common(g)
    seg = draw_seg(g, total)
    lam = bwd_lambdas(g, H)
    S = len(lens)
    say("case pair varlen %d: lens=%s H=%d d=%d %s block=%d seg=%d"
        % (case, lens, H, d, dtype, block, seg))
    q, k, v = inputs.host_qkv((H, total, d), 24100 + case, dtype=dtype)
    do, _, _ = inputs.host_qkv((H, total, d), 24101 + case, dtype=dtype)
    init = inputs.host_state((S, H, d, d), 24102 + case)
    dfin = inputs.host_state((S, H, d, d), 24103 + case)
    tq, tk, tv, tdo = (dev(x, dtype) for x in (q, k, v, do))
    tl, ti, tc = dev(lam, "fp32"), dev(init, "fp32"), dev_i32(cu)
    out, fin, saved = la.lightning_attn_fwd_varlen_save(tq, tk, tv, tl, tc, block=block,
                                                        init_states=ti, segment_tokens=seg)
    dq, dk, dv, dinit = la.lightning_attn_bwd_varlen_saved(tq, tk, tv, tl, tdo, tc, saved,
                                                           block=block,
                                                           dfinals=dev(dfin, "fp32"),
                                                           init_states=ti, segment_tokens=seg)
    sync()
    o_ref, f_ref, _ = oracle.fwd_varlen(q, k, v, lam, cu, init=init)
    ref = oracle_bwd_packed(cu, q, k, v, lam, do, dfin, init)
    errs = [rel_err(host(out), o_ref), rel_err(host(fin), f_ref)]
    errs += [rel_err(host(a), b) for a, b in zip((dq, dk, dv, dinit), ref)]
    say("   err out %.3e state %.3e dq %.3e dk %.3e dv %.3e dinit %.3e" % tuple(errs))
    assert max(errs) <= TOL[dtype]


# ---------------------------------------------------------------------------
# prefix-state snapshots

SNAP_CASES = 5


@pytest.mark.parametrize("case", range(SNAP_CASES))
def test_random_snapshots(case):
    g = np.random.default_rng(25000 + case)
    H = int(g.integers(1, 4))
    lens = draw_lens(g, 5)
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    d, dtype, block = draw_common(g)
    seg = draw_seg(g, total)
    # (an interval of 1 stores a state per token: only for short batches)
    iv = int(g.choice([1, 7, 64] if total <= 400 else [64, 128, 200, 256]))
    with_init = bool(g.integers(0, 2))
    lam = draw_decays(g, H)
    S = len(lens)
    say("case snapshots %d: lens=%s H=%d d=%d %s block=%d seg=%d interval=%d init=%s"
        % (case, lens, H, d, dtype, block, seg, iv, with_init))
    q, k, v = inputs.host_qkv((H, total, d), 25100 + case, dtype=dtype)
    init = inputs.host_state((S, H, d, d), 25101 + case) if with_init else None
    out, fin, snaps, offs = la.lightning_attn_fwd_varlen_snapshots(
        dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(lam, "fp32"), dev_i32(cu), iv,
        block=block, init_states=None if init is None else dev(init, "fp32"),
        segment_tokens=seg)
    sync()
    o_ref, f_ref, s_ref, off_ref = oracle.fwd_varlen_snapshots(q, k, v, lam, cu, iv, init=init)
    assert np.array_equal(offs.cpu().numpy(), off_ref)
    errs = [rel_err(host(out), o_ref), rel_err(host(fin), f_ref), rel_err(host(snaps), s_ref)]
    say("   rows %d err out %.3e state %.3e snapshots %.3e" % ((s_ref.shape[0],) + tuple(errs)))
    assert max(errs) <= TOL[dtype]


# ---------------------------------------------------------------------------
# decode steps

DECODE_CASES = 5


@pytest.mark.parametrize("case", range(DECODE_CASES))
def test_random_decode(case):
    g = np.random.default_rng(26000 + case)
    B, H = int(g.integers(1, 6)), int(g.integers(1, 5))
    d = int(g.choice([64, 128]))
    dtype = str(g.choice(["bf16", "fp32"]))
    steps = int(g.integers(1, 9))
    lam = draw_decays(g, H)
    say("case decode %d: B=%d H=%d d=%d %s steps=%d" % (case, B, H, d, dtype, steps))
    q, k, v = inputs.host_qkv((steps, B, H, d), 26100 + case, dtype=dtype)
    st0 = inputs.host_state((B, H, d, d), 26101 + case)
    state = dev(st0, "fp32")
    ref_state = st0.astype(np.float64).copy()
    tl = dev(lam, "fp32")
    for t in range(steps):
        out = la.lightning_attn_decode(dev(q[t], dtype), dev(k[t], dtype), dev(v[t], dtype), tl,
                                       state)
        sync()
        o_ref, _ = oracle.decode(q[t], k[t], v[t], lam, ref_state)
        eo = rel_err(host(out), o_ref)
        assert eo <= TOL[dtype], (t, eo)
    es = rel_err(host(state), ref_state)
    say("   err last out %.3e state %.3e" % (eo, es))
    assert es <= TOL[dtype]


DECODE_CH_CASES = 3


@pytest.mark.parametrize("case", range(DECODE_CH_CASES))
def test_random_decode_chdecay(case):
    """A channel-wise decode step from state S equals the first output row
    and final state of a one-token channel-wise prefill from S."""
    g = np.random.default_rng(27000 + case)
    B, H = int(g.integers(1, 6)), int(g.integers(1, 5))
    d = int(g.choice([64, 128]))
    dtype = str(g.choice(["bf16", "fp32"]))
    alpha = np.exp(-np.exp2(g.uniform(-10, 2, (H, d)))).astype(np.float32)
    say("case decode chdecay %d: B=%d H=%d d=%d %s" % (case, B, H, d, dtype))
    q, k, v = inputs.host_qkv((B, H, d), 27100 + case, dtype=dtype)
    st0 = inputs.host_state((B, H, d, d), 27101 + case)
    state = dev(st0, "fp32")
    out = la.lightning_attn_decode_chdecay(dev(q, dtype), dev(k, dtype), dev(v, dtype),
                                           dev(alpha, "fp32"), state)
    sync()
    o_ref, f_ref = oracle.fwd_chdecay(q[:, :, None], k[:, :, None], v[:, :, None], alpha,
                                      init=st0)
    eo, es = rel_err(host(out), o_ref[:, :, 0]), rel_err(host(state), f_ref)
    say("   err out %.3e state %.3e" % (eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


# ---------------------------------------------------------------------------
# allocation-free prefill

NOALLOC_CASES = 4


@pytest.mark.parametrize("case", range(NOALLOC_CASES))
def test_random_noalloc(case):
    g = np.random.default_rng(28000 + case)
    B, H = int(g.integers(1, 3)), int(g.integers(1, 5))
    N = int(g.integers(1, 1500))
    d, dtype, block = draw_common(g)
    seg = draw_seg(g, N)
    with_init = bool(g.integers(0, 2))
    lam = draw_decays(g, H)
    say("case noalloc %d: B=%d H=%d N=%d d=%d %s block=%d seg=%d init=%s"
        % (case, B, H, N, d, dtype, block, seg, with_init))
    q, k, v = inputs.host_qkv((B, H, N, d), 28100 + case, dtype=dtype)
    init = inputs.host_state((B, H, d, d), 28101 + case) if with_init else None
    out, fin = la.lightning_attn_fwd_noalloc(dev(q, dtype), dev(k, dtype), dev(v, dtype),
                                             dev(lam, "fp32"), block=block,
                                             init_state=None if init is None else dev(init, "fp32"),
                                             segment_tokens=seg)
    sync()
    o_ref, f_ref, _ = oracle.fwd(q, k, v, lam, init=init)
    eo, ef = rel_err(host(out), o_ref), rel_err(host(fin), f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


# ---------------------------------------------------------------------------
# token-major packed prefill

TM_VARLEN_CASES = 4


@pytest.mark.parametrize("case", range(TM_VARLEN_CASES))
def test_random_varlen_token_major(case):
    g = np.random.default_rng(29000 + case)
    H = int(g.integers(1, 5))
    lens = draw_lens(g, 6)
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    d, dtype, block = draw_common(g)
    seg = draw_seg(g, total)
    with_init = bool(g.integers(0, 2))
    lam = draw_decays(g, H)
    S = len(lens)
    say("case varlen token-major %d: lens=%s H=%d d=%d %s block=%d seg=%d init=%s"
        % (case, lens, H, d, dtype, block, seg, with_init))
    q, k, v = inputs.host_qkv((H, total, d), 29100 + case, dtype=dtype)
    init = inputs.host_state((S, H, d, d), 29101 + case) if with_init else None
    tq, tk, tv = (to_token_major(dev(x, dtype)) for x in (q, k, v))
    out, fin = la.lightning_attn_fwd_varlen_layout(
        tq, tk, tv, dev(lam, "fp32"), dev_i32(cu), la.LA_TOKEN_MAJOR, block=block,
        init_states=None if init is None else dev(init, "fp32"), segment_tokens=seg)
    sync()
    o_ref, f_ref, _ = oracle.fwd_varlen(q, k, v, lam, cu, init=init)
    eo, ef = rel_err(host(out.transpose(0, 1)), o_ref), rel_err(host(fin), f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


# ---------------------------------------------------------------------------
# mixed serving step

MIXED_CASES = 4


@pytest.mark.parametrize("case", range(MIXED_CASES))
def test_random_mixed_step(case):
    torch = torch_mod()
    g = np.random.default_rng(30000 + case)
    H = int(g.integers(1, 5))
    lens = draw_lens(g, 4)
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    d, dtype, block = draw_common(g)
    seg = draw_seg(g, total)
    Bd = int(g.integers(1, 7))
    two = bool(g.integers(0, 2))
    lam = draw_decays(g, H)
    S = len(lens)
    say("case mixed %d: lens=%s decode B=%d H=%d d=%d %s block=%d seg=%d two_streams=%s"
        % (case, lens, Bd, H, d, dtype, block, seg, two))
    q, k, v = inputs.host_qkv((H, total, d), 30100 + case, dtype=dtype)
    init = inputs.host_state((S, H, d, d), 30101 + case)
    dq_, dk_, dv_ = inputs.host_qkv((Bd, H, d), 30102 + case, dtype=dtype)
    st0 = inputs.host_state((Bd, H, d, d), 30103 + case)
    state = dev(st0, "fp32")
    side = torch.cuda.Stream() if two else None
    tqkv = (dev(q, dtype), dev(k, dtype), dev(v, dtype))
    tdec = (dev(dq_, dtype), dev(dk_, dtype), dev(dv_, dtype))
    tl, ti, tc = dev(lam, "fp32"), dev(init, "fp32"), dev_i32(cu)
    torch.cuda.synchronize()  # inputs made on this stream are read on the other one
    pout, fin, dout = la.lightning_attn_mixed_step(
        tl, tqkv, tc, tdec, state, block=block, init_states=ti, segment_tokens=seg,
        decode_stream=side)
    torch.cuda.synchronize()
    o_ref, f_ref, _ = oracle.fwd_varlen(q, k, v, lam, cu, init=init)
    ref_state = st0.astype(np.float64).copy()
    d_ref, _ = oracle.decode(dq_, dk_, dv_, lam, ref_state)
    errs = [rel_err(host(pout), o_ref), rel_err(host(fin), f_ref), rel_err(host(dout), d_ref),
            rel_err(host(state), ref_state)]
    say("   err prefill out %.3e states %.3e decode out %.3e state %.3e" % tuple(errs))
    assert max(errs) <= TOL[dtype]
