"""GPU parity: the HIP path (through the C ABI, via the Python binding)
against the double-precision CPU oracle, on the same seeded inputs.

Bar (max |o - o_ref| / max |o_ref| over the compared set, and the same for
the final state): <= 1e-4 for float32 inputs, <= 2e-2 for bf16 inputs.
Every test compares every element of what it checks; the full-size
workloads run in the launch configuration the benchmark times.  (Only the
tests past 2^31 elements compare windows, each exact in double; see there.)
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


@pytest.fixture(params=["auto", "phased", "fused"])
def prefill_path(request, monkeypatch):
    """Runs a test once per prefill path: the library's own choice, the
    three-phase segment scan, and the single-pass kernel (bf16, d = 128)."""
    if request.param == "auto":
        monkeypatch.delenv("LIGHTNING_ATTN_PREFILL", raising=False)
    else:
        monkeypatch.setenv("LIGHTNING_ATTN_PREFILL", request.param)
    return request.param


def torch_mod():
    import torch
    return torch


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    torch = torch_mod()
    return t.detach().to(torch.float32).cpu().numpy()


def dev_inputs(shape, seed, dtype):
    """Seeded host inputs (numpy), copied to the GPU in the compute dtype."""
    torch = torch_mod()
    q, k, v = inputs.host_qkv(shape, seed, dtype=dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return [torch.from_numpy(x).to("cuda").to(tdt) for x in (q, k, v)], (q, k, v)


def run_fwd_case(B, H, N, d, dtype, seed, block=128, seg=0, with_init=False, lam=None,
                 token_major=False):
    torch = torch_mod()
    say("case fwd B=%d H=%d N=%d d=%d %s seg=%d init=%s token_major=%s"
        % (B, H, N, d, dtype, seg, with_init, token_major))
    (tq, tk, tv), (q, k, v) = dev_inputs((B, H, N, d), seed, dtype)
    lam = inputs.decay_schedule(H) if lam is None else np.asarray(lam, np.float32)
    tl = torch.from_numpy(lam).to("cuda")
    init = inputs.host_state((B, H, d, d), seed + 1) if with_init else None
    ti = torch.from_numpy(init).to("cuda") if with_init else None
    if token_major:
        # [B, N, H, d] copies; out starts as NaN so that an unwritten (or
        # wrongly addressed) element fails the finiteness check below.
        tq, tk, tv = (t.transpose(1, 2).contiguous() for t in (tq, tk, tv))
        out = torch.full_like(tq, float("nan"))
        out, fin = la.lightning_attn_fwd_layout(tq, tk, tv, tl, la.LA_TOKEN_MAJOR, block=block,
                                                init_state=ti, segment_tokens=seg, out=out)
        out = out.transpose(1, 2)
    else:
        out, fin = la.lightning_attn_fwd(tq, tk, tv, tl, block=block, init_state=ti,
                                         segment_tokens=seg)
    torch.cuda.synchronize()
    o_ref, f_ref, _ = oracle.fwd(q, k, v, lam, init=init)
    eo, ef = rel_err(host(out), o_ref), rel_err(host(fin), f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert np.isfinite(host(out)).all()
    assert eo <= TOL[dtype] and ef <= TOL[dtype], (eo, ef)
    return host(out), host(fin), (q, k, v)


def test_tiny_fp32_workload():
    """B=1 H=2 N=256 d=64 block=64, float32: every element."""
    run_fwd_case(1, 2, 256, 64, "fp32", seed=1, block=64)


def test_mid_bf16_workload():
    """B=2 H=8 N=4096 d=128 block=64, bf16: every element."""
    run_fwd_case(2, 8, 4096, 128, "bf16", seed=2, block=64)


@pytest.mark.parametrize("seg", [4096, 128, 640, 1000, 8192, la.LA_SEGMENT_PER_SEQUENCE])
def test_segment_split_invariance_bf16(seg, prefill_path):
    """Any cut of the token axis into segments (on-device LASP+ scan) gives
    the oracle's result: segments of one block, ragged segments, segments
    spanning two sequences."""
    run_fwd_case(2, 4, 4096, 128, "bf16", seed=20, seg=seg)


@pytest.mark.parametrize("N", [1, 2, 127, 128, 129, 300, 1000])
def test_ragged_tails_bf16(N, prefill_path):
    run_fwd_case(2, 3, N, 128, "bf16", seed=30 + N, with_init=True,
                 lam=[0.9961, 0.3997, 0.75])


@pytest.mark.parametrize("d,dtype", [(64, "fp32"), (128, "fp32"), (64, "bf16")])
@pytest.mark.parametrize("N,seg", [(300, 0), (300, 64), (77, 0)])
def test_vector_alu_paths(d, dtype, N, seg):
    run_fwd_case(1, 3, N, d, dtype, seed=40 + N + d, seg=seg, with_init=True,
                 lam=[0.999, 0.5, 0.9])


@pytest.mark.parametrize("dtype,d,seg", [("bf16", 128, 2048), ("bf16", 128, 4096),
                                         ("fp32", 64, 1024)])
def test_local_state_zero_weight_chunks(dtype, d, seg, prefill_path):
    """Local-state passes skip leading chunks whose decay weights are below
    2^-160 (exactly zero in float32).  The decays put that cut inside the
    segments for some heads (0.3, 0.8, 0.93) and beyond them for others, so a
    misplaced cut changes the entering states and fails the comparison."""
    run_fwd_case(1, 6, 6000, d, dtype, seed=60 + d, seg=seg, with_init=True,
                 lam=[0.3, 0.8, 0.93, 0.97, 0.99, 0.999])


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "fp32")])
def test_decay_one_across_segments(d, dtype, prefill_path):
    """lambda = 1 exactly (plain causal linear attention) in heads whose
    sequences cross segment cuts: no token of a local-state pass may be
    skipped as weightless."""
    run_fwd_case(1, 3, 3000, d, dtype, seed=65 + d, seg=1024, with_init=True,
                 lam=[1.0, 0.9, 1.0])


def test_tied_decays_across_heads(prefill_path):
    """The local-state pass hands out the heads' first pieces in order of
    decreasing decay, ties broken by head index: heads with equal decays
    (three groups of four here, several segments and pieces each) must each
    still get every piece computed exactly once."""
    run_fwd_case(1, 12, 20000, 128, "bf16", seed=71, seg=4096, with_init=True,
                 lam=[0.99] * 4 + [0.9] * 4 + [0.999] * 4)


def test_initial_state_bf16(prefill_path):
    run_fwd_case(1, 4, 2048, 128, "bf16", seed=50, with_init=True, seg=512)
    run_fwd_case(2, 40, 1500, 128, "bf16", seed=51, with_init=True)


def test_zero_length_returns_initial_state():
    torch = torch_mod()
    B, H, d = 2, 3, 128
    init = torch.randn(B, H, d, d, device="cuda")
    q = torch.empty(B, H, 0, d, device="cuda", dtype=torch.bfloat16)
    out, fin = la.lightning_attn_fwd(q, q.clone(), q.clone(),
                                     torch.from_numpy(inputs.decay_schedule(H)).cuda(),
                                     init_state=init)
    torch.cuda.synchronize()
    assert torch.equal(fin, init)
    out, fin = la.lightning_attn_fwd(q, q.clone(), q.clone(),
                                     torch.from_numpy(inputs.decay_schedule(H)).cuda())
    torch.cuda.synchronize()
    assert torch.count_nonzero(fin).item() == 0


def test_deterministic_bitwise(prefill_path):
    torch = torch_mod()
    (tq, tk, tv), _ = dev_inputs((1, 48, 8192, 128), 60, "bf16")
    tl = torch.from_numpy(inputs.decay_schedule(48)).cuda()
    o1, f1 = la.lightning_attn_fwd(tq, tk, tv, tl)
    o2, f2 = la.lightning_attn_fwd(tq, tk, tv, tl)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("low_word", [0x40000000, 0x80000100, 0xFFFF4000])
def test_tile_addresses_any_low_word(low_word, prefill_path):
    """K and V placed so that the low 32 bits of their addresses sit below
    2^31, at or above it, and 48 KiB under 2^32 (the second 128-token chunk
    of head 0 then straddles a 4 GiB line).  The tile loads form a 64-bit
    base plus a 32-bit lane offset, which must neither sign-extend the low
    word nor wrap at 4 GiB.  The outputs must be bit-identical to the same
    inputs in ordinary allocations (and within the oracle bar)."""
    torch = torch_mod()
    B, H, N, d = 1, 2, 2048, 128
    (tq, tk, tv), (q, k, v) = dev_inputs((B, H, N, d), 70, "bf16")
    tl = torch.from_numpy(inputs.decay_schedule(H)).cuda()
    o_ref, f_ref = la.lightning_attn_fwd(tq, tk, tv, tl)
    n = tk.numel()
    pool = torch.empty((1 << 32) + (64 << 20), dtype=torch.uint8, device="cuda")
    off = (low_word - pool.data_ptr()) % (1 << 32)
    say("case tile addresses: k at low word %#x (pool offset %d)" % (low_word, off))
    flat = pool[off:off + 4 * n + 8192].view(torch.bfloat16)
    pk = flat[:n].view(B, H, N, d)
    pv = flat[n + 2048:2 * n + 2048].view(B, H, N, d)
    pk.copy_(tk)
    pv.copy_(tv)
    assert pk.data_ptr() & 0xFFFFFFFF == low_word
    out, fin = la.lightning_attn_fwd(tq, pk, pv, tl)
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(fin, f_ref)
    o_or, f_or, _ = oracle.fwd(q, k, v, inputs.decay_schedule(H))
    assert rel_err(host(out), o_or) <= TOL["bf16"] and rel_err(host(fin), f_or) <= TOL["bf16"]
    del pool, flat, pk, pv


# ------------------------------------------------------------------ varlen


def run_varlen_case(lens, H, d, dtype, seed, seg=0, with_init=True, token_major=False, lam=None):
    torch = torch_mod()
    say("case varlen lens=%s H=%d d=%d %s seg=%d token_major=%s"
        % (lens[:8], H, d, dtype, seg, token_major))
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    (tq, tk, tv), (q, k, v) = dev_inputs((H, total, d), seed, dtype)
    lam = inputs.decay_schedule(H) if lam is None else np.asarray(lam, np.float32)
    init = inputs.host_state((len(lens), H, d, d), seed + 1) if with_init else None
    ti = torch.from_numpy(init).cuda() if with_init else None
    if token_major:
        tq, tk, tv = (t.transpose(0, 1).contiguous() for t in (tq, tk, tv))  # [total, H, d]
        out = torch.full_like(tq, float("nan"))
        out, fin = la.lightning_attn_fwd_varlen_layout(
            tq, tk, tv, torch.from_numpy(lam).cuda(), torch.from_numpy(cu).cuda(),
            la.LA_TOKEN_MAJOR, init_states=ti, segment_tokens=seg, out=out)
        out = out.transpose(0, 1)
        assert bool(torch.isfinite(out).all())
    else:
        out, fin = la.lightning_attn_fwd_varlen(tq, tk, tv, torch.from_numpy(lam).cuda(),
                                                torch.from_numpy(cu).cuda(), init_states=ti,
                                                segment_tokens=seg)
    torch.cuda.synchronize()
    o_ref, f_ref, _ = oracle.fwd_varlen(q, k, v, lam, cu, init=init)
    eo = rel_err(host(out), o_ref) if total else 0.0
    ef = rel_err(host(fin), f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL[dtype] and ef <= TOL[dtype], (eo, ef)
    return host(out), host(fin), (q, k, v), cu


@pytest.mark.parametrize("B,H,N,d,dtype,seg", [
    (2, 5, 1000, 128, "bf16", 0), (2, 5, 1000, 128, "bf16", 256), (1, 3, 4099, 128, "bf16", 1024),
    (2, 3, 300, 64, "fp32", 0), (2, 3, 300, 128, "fp32", 96), (1, 4, 333, 64, "bf16", 0)])
def test_token_major_layout(B, H, N, d, dtype, seg, prefill_path):
    """[B, N, H, d] inputs and outputs (a projection's layout, read in place):
    the oracle's result for every element, heads interleaved in each row,
    every output element written."""
    run_fwd_case(B, H, N, d, dtype, seed=110 + N + d, seg=seg, with_init=True,
                 token_major=True)


@pytest.mark.parametrize("d,dtype,seg", [(128, "bf16", 0), (128, "bf16", 200), (64, "fp32", 0)])
def test_varlen_token_major_layout(d, dtype, seg, prefill_path):
    run_varlen_case([300, 0, 1, 129, 1024, 5, 0, 640, 2000], 4, d, dtype, seed=120 + d, seg=seg,
                    token_major=True)


@pytest.mark.parametrize("seg", [0, 128, 200, 100000, la.LA_SEGMENT_PER_SEQUENCE])
def test_varlen_bf16(seg, prefill_path):
    run_varlen_case([300, 0, 1, 129, 1024, 5, 0, 640, 2000], 4, 128, "bf16", seed=70, seg=seg)


@pytest.mark.parametrize("seg", [4096, 16384, 32768])
def test_varlen_many_pieces(seg, prefill_path):
    """Segments of 4096, 16384 and 32768 tokens: the local-state pass cuts the
    weighted part of each segment's last piece into 4, 8 and 16 parts for the
    slowest head (fewer for the faster ones) whose weighted sum the scan
    forms; the sequences cross the segment cuts, so every part's weight
    reaches an entering state."""
    run_varlen_case([20000, 0, 3000, 37000, 100, 4500], 3, 128, "bf16", seed=72, seg=seg)


@pytest.mark.parametrize("d,dtype", [(64, "fp32"), (128, "fp32"), (64, "bf16")])
@pytest.mark.parametrize("seg", [48, la.LA_SEGMENT_PER_SEQUENCE])
def test_varlen_vector_alu(d, dtype, seg):
    run_varlen_case([33, 0, 64, 1, 100], 2, d, dtype, seed=71, seg=seg)


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "fp32")])
def test_varlen_one_segment_per_sequence(d, dtype):
    """LA_SEGMENT_PER_SEQUENCE: one workgroup per (sequence, head) and the
    output pass alone; empty sequences (first, inside, last) get their initial
    state as final state from it, with and without initial states."""
    lens = [0, 300, 0, 1, 129, 2000, 5, 0]
    run_varlen_case(lens, 3, d, dtype, seed=73, seg=la.LA_SEGMENT_PER_SEQUENCE)
    run_varlen_case(lens, 3, d, dtype, seed=74, seg=la.LA_SEGMENT_PER_SEQUENCE, with_init=False)
    run_varlen_case(lens, 3, d, dtype, seed=75, seg=la.LA_SEGMENT_PER_SEQUENCE, token_major=True)


@pytest.mark.parametrize("seg", [0, la.LA_SEGMENT_PER_SEQUENCE])
def test_varlen_all_empty(seg):
    torch = torch_mod()
    H, d = 2, 128
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    q = torch.empty(H, 0, d, dtype=torch.bfloat16, device="cuda")
    init = torch.randn(3, H, d, d, device="cuda")
    out, fin = la.lightning_attn_fwd_varlen(q, q.clone(), q.clone(),
                                            torch.from_numpy(inputs.decay_schedule(H)).cuda(), cu,
                                            init_states=init, segment_tokens=seg)
    torch.cuda.synchronize()
    assert torch.equal(fin, init)


# ------------------------------------------------------- slow decay
# Heads with lambda <= 2^-15 take the kernels' per-power branch (every power
# of lambda exponentiated on its own, where the fast branch factors powers
# into one exponential per group of 8 times per-head constants), in the chunk
# loop, the state update, the local-state pass and the single-pass kernel.
# They run here beside ordinary heads in one call.  As lambda -> 0 the
# recurrence reduces to o_t = (q_t . k_t) v_t and S = k_{N-1}^T v_{N-1}
# (MiniMax-01 report, section 2.2.1, with the decay of section 3.2.2): the
# heads at 1e-6 and 1e-20 are also checked against that closed form, which
# they meet to within lambda (far below the bar).

SLOW_LAM = [0.9, 2.0 ** -16, 1e-6, 1e-20, 0.5, 0.999]
ZERO_HEADS = (2, 3)   # lambda 1e-6 and 1e-20


def lambda_zero_err(o, q, k, v, fin=None):
    """Error of outputs o [..., N, d] (and final state fin [..., d, d])
    against the lambda -> 0 closed form, in double."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    o_cf = np.sum(q * k, axis=-1, keepdims=True) * v
    e = rel_err(o, o_cf)
    if fin is not None:
        s_cf = k[..., -1, :, None] * v[..., -1, None, :]
        e = max(e, rel_err(fin, s_cf))
    return e


@pytest.mark.parametrize("seg", [1024, 0])
def test_slow_decay_fixed(seg, prefill_path):
    """Fixed-length prefill over 3000 tokens with an initial state: segment
    cuts (so the local-state pass, the scan or the single-pass hand-offs see
    the slow heads) and the library's own plan."""
    o, f, (q, k, v) = run_fwd_case(1, len(SLOW_LAM), 3000, 128, "bf16", seed=140 + seg, seg=seg,
                                   with_init=True, lam=SLOW_LAM)
    for h in ZERO_HEADS:
        e = lambda_zero_err(o[:, h], q[:, h], k[:, h], v[:, h], f[:, h])
        say("   head %d (lambda %g) closed-form err %.3e" % (h, SLOW_LAM[h], e))
        assert e <= TOL["bf16"], e


@pytest.mark.parametrize("N", [1, 129])
def test_slow_decay_ragged_and_fp32(N):
    """Ragged tails on the MFMA path, and the float32 vector-ALU path."""
    run_fwd_case(2, len(SLOW_LAM), N, 128, "bf16", seed=150 + N, with_init=True, lam=SLOW_LAM)
    run_fwd_case(1, len(SLOW_LAM), 300 + N, 64, "fp32", seed=152 + N, seg=128, with_init=True,
                 lam=SLOW_LAM)


@pytest.mark.parametrize("seg", [200, la.LA_SEGMENT_PER_SEQUENCE])
def test_slow_decay_varlen(seg, prefill_path):
    """Packed sequences (empty ones included) with the slow heads."""
    lens = [300, 0, 1, 129, 1024, 5, 640]
    o, f, (q, k, v), cu = run_varlen_case(lens, len(SLOW_LAM), 128, "bf16", seed=160, seg=seg,
                                          lam=SLOW_LAM)
    for h in ZERO_HEADS:
        worst = 0.0
        for j in range(len(lens)):
            a, b = int(cu[j]), int(cu[j + 1])
            if b > a:
                worst = max(worst, lambda_zero_err(o[h, a:b], q[h, a:b], k[h, a:b], v[h, a:b],
                                                   f[j, h]))
        say("   head %d (lambda %g) closed-form err %.3e" % (h, SLOW_LAM[h], worst))
        assert worst <= TOL["bf16"], worst


def test_slow_decay_decode():
    """Decode steps with the slow heads: each step's output is, as lambda ->
    0, (q . k) v of that step alone."""
    torch = torch_mod()
    B, H, d, steps = 3, len(SLOW_LAM), 128, 6
    (tq, tk, tv), (q, k, v) = dev_inputs((steps, B, H, d), 170, "bf16")
    lam = np.asarray(SLOW_LAM, np.float32)
    S0 = inputs.host_state((B, H, d, d), 171)
    st = torch.from_numpy(S0).cuda()
    tl = torch.from_numpy(lam).cuda()
    S = S0.astype(np.float64)
    worst = worst_cf = 0.0
    for t in range(steps):
        o = host(la.lightning_attn_decode(tq[t], tk[t], tv[t], tl, st))
        o_ref, _ = oracle.decode(q[t], k[t], v[t], lam, S)
        worst = max(worst, rel_err(o, o_ref))
        for h in ZERO_HEADS:
            worst_cf = max(worst_cf, lambda_zero_err(o[:, h, None], q[t][:, h, None],
                                                     k[t][:, h, None], v[t][:, h, None]))
    torch.cuda.synchronize()
    es = rel_err(host(st), S)
    say("   err out %.3e state %.3e closed form %.3e" % (worst, es, worst_cf))
    assert max(worst, es, worst_cf) <= TOL["bf16"]


# ------------------------------------------------------------------ decode


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "bf16"), (128, "fp32"), (64, "fp32")])
def test_decode_steps(d, dtype):
    torch = torch_mod()
    B, H, steps = 3, 4, 12
    say("case decode B=%d H=%d d=%d %s" % (B, H, d, dtype))
    (tq, tk, tv), (q, k, v) = dev_inputs((steps, B, H, d), 80 + d, dtype)
    lam = inputs.decay_schedule(H)
    S0 = inputs.host_state((B, H, d, d), 81)
    st = torch.from_numpy(S0).cuda()
    tl = torch.from_numpy(lam).cuda()
    S = S0.astype(np.float64)
    worst = 0.0
    for t in range(steps):
        o = la.lightning_attn_decode(tq[t], tk[t], tv[t], tl, st)
        o_ref, _ = oracle.decode(q[t], k[t], v[t], lam, S)
        worst = max(worst, rel_err(host(o), o_ref))
    torch.cuda.synchronize()
    es = rel_err(host(st), S)
    say("   err out %.3e state %.3e" % (worst, es))
    assert worst <= TOL[dtype] and es <= TOL[dtype]


def test_decode_matches_prefill_rows():
    """Decoding token t from the prefill state after t tokens reproduces
    prefill row t (recurrent form, eq. 12)."""
    torch = torch_mod()
    B, H, N, d = 2, 4, 200, 128
    (tq, tk, tv), _ = dev_inputs((B, H, N + 1, d), 90, "bf16")
    tl = torch.from_numpy(inputs.decay_schedule(H)).cuda()
    out, fin = la.lightning_attn_fwd(tq[:, :, :N].contiguous(), tk[:, :, :N].contiguous(),
                                     tv[:, :, :N].contiguous(), tl)
    full, _ = la.lightning_attn_fwd(tq, tk, tv, tl)
    o = la.lightning_attn_decode(tq[:, :, N].contiguous(), tk[:, :, N].contiguous(),
                                 tv[:, :, N].contiguous(), tl, fin)
    torch.cuda.synchronize()
    assert rel_err(host(o), host(full[:, :, N])) < 2e-2


# ------------------------------------------------- full-size workloads
# Same sizes, seeds and launch configuration as bench.py; inputs drawn on
# the GPU (seeded Philox) and copied back for the oracle.  Every element of
# every output and final state is compared (whole_rel_err), the oracle's
# result cached across the prefill paths that share it.


def _layer_ref():
    """Oracle output and final states of the B=1 H=64 N=32768 workload."""
    w = inputs.WORKLOADS["layer_h64_n32k"]

    def compute():
        tq, tk, tv = inputs.device_qkv((w["B"], w["H"], w["N"], w["d"]), w["seed"], "bf16")
        q, k, v = host(tq), host(tk), host(tv)
        del tq, tk, tv
        o_ref, f_ref, _ = oracle.fwd(q, k, v, inputs.decay_schedule(w["H"]))
        return o_ref, f_ref

    return ORACLE_CACHE.get("layer_h64_n32k", compute)


def test_full_layer_h64_n32k(prefill_path):
    """B=1 H=64 N=32768 d=128 block=128: every output element and every
    final-state entry of all 64 heads against the oracle's recurrence."""
    torch = torch_mod()
    w = inputs.WORKLOADS["layer_h64_n32k"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    say("case full layer_h64_n32k path=%s" % prefill_path)
    tq, tk, tv = inputs.device_qkv((B, H, N, d), w["seed"], "bf16")
    lam = inputs.decay_schedule(H)
    out, fin = la.lightning_attn_fwd(tq, tk, tv, torch.from_numpy(lam).cuda(), block=w["block"])
    torch.cuda.synchronize()
    del tq, tk, tv
    o_ref, f_ref = _layer_ref()
    eo = whole_rel_err(out, o_ref, dim=1, name="out")
    ef = whole_rel_err(fin, f_ref, dim=1, name="final_state")
    say("   err out %.3e state %.3e (all %d heads)" % (eo, ef, H))
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


def test_full_layer_h64_n32k_token_major(prefill_path):
    """The headline workload in [B, N, H, d] layout: bit-identical to the
    head-major call (the same arithmetic, only the addressing differs), and
    every element against the oracle."""
    torch = torch_mod()
    w = inputs.WORKLOADS["layer_h64_n32k"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    say("case full layer_h64_n32k token-major path=%s" % prefill_path)
    tq, tk, tv = inputs.device_qkv((B, H, N, d), w["seed"], "bf16")
    tl = torch.from_numpy(inputs.decay_schedule(H)).cuda()
    out_h, fin_h = la.lightning_attn_fwd(tq, tk, tv, tl, block=w["block"])
    tq, tk, tv = (t.transpose(1, 2).contiguous() for t in (tq, tk, tv))
    out_t, fin_t = la.lightning_attn_fwd_layout(tq, tk, tv, tl, la.LA_TOKEN_MAJOR,
                                                block=w["block"])
    torch.cuda.synchronize()
    del tq, tk, tv
    assert torch.equal(out_t.transpose(1, 2), out_h) and torch.equal(fin_t, fin_h)
    del out_h, fin_h
    o_ref, f_ref = _layer_ref()
    eo = whole_rel_err(out_t, o_ref.transpose(0, 2, 1, 3), dim=2, name="out")
    ef = whole_rel_err(fin_t, f_ref, dim=1, name="final_state")
    say("   err out %.3e state %.3e (all %d heads)" % (eo, ef, H))
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


def test_full_varlen_h64_65536(prefill_path):
    """65536 packed tokens, lognormal lengths, H=64: every output element of
    every sequence and head, and every final state, against the oracle's
    packed recurrence."""
    torch = torch_mod()
    w = inputs.WORKLOADS["layer_h64_varlen64k"]
    H, total, d = w["H"], w["total"], w["d"]
    lens = inputs.varlen_lengths(total=total, seed=w["seed"])
    cu = inputs.cu_seqlens(lens)
    say("case full varlen: %d sequences, max %d, path=%s" % (len(lens), max(lens), prefill_path))
    tq, tk, tv = inputs.device_qkv((H, total, d), w["seed"], "bf16")
    lam = inputs.decay_schedule(H)
    out, fin = la.lightning_attn_fwd_varlen(tq, tk, tv, torch.from_numpy(lam).cuda(),
                                            torch.from_numpy(cu).cuda(), block=w["block"])
    torch.cuda.synchronize()

    def compute():
        o_ref, f_ref, _ = oracle.fwd_varlen(host(tq), host(tk), host(tv), lam, cu)
        return o_ref, f_ref

    o_ref, f_ref = ORACLE_CACHE.get("layer_h64_varlen64k", compute)
    eo = whole_rel_err(out, o_ref, dim=0, name="out")
    ef = whole_rel_err(fin, f_ref, dim=0, name="final_states")
    say("   err out %.3e state %.3e (all %d sequences, all %d heads)" % (eo, ef, len(lens), H))
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


def test_full_million_h8():
    """B=1 H=8 N=1048576 d=128 block=256 (4096 blocks carried in one
    sequence): every output element and final-state entry of all 8 heads
    against the oracle's recurrence over the whole sequence."""
    torch = torch_mod()
    w = inputs.WORKLOADS["million_h8"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    say("case full million_h8")
    tq, tk, tv = inputs.device_qkv((B, H, N, d), w["seed"], "bf16")
    lam = inputs.decay_schedule(H)
    out, fin = la.lightning_attn_fwd(tq, tk, tv, torch.from_numpy(lam).cuda(), block=w["block"])
    torch.cuda.synchronize()
    ORACLE_CACHE.clear()  # release any cached reference first
    q, k, v = host(tq), host(tk), host(tv)
    del tq, tk, tv
    o_ref, f_ref, used = oracle.fwd(q, k, v, lam)
    del q, k, v
    eo = whole_rel_err(out, o_ref, dim=1, name="out")
    ef = whole_rel_err(fin, f_ref, dim=1, name="final_state")
    say("   err out %.3e state %.3e (all %d heads, %d oracle threads)" % (eo, ef, H, used))
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


def test_full_decode_b128_h64():
    """128 sequences x 64 heads, d=128, 256 consecutive steps from a
    N(0, 0.1^2) state: every output of every (sequence, head) pair at every
    step, and the whole final state, against the oracle stepped alongside."""
    torch = torch_mod()
    w = inputs.WORKLOADS["decode_b128_h64"]
    B, H, d, T = w["B"], w["H"], w["d"], w["steps"]
    say("case full decode_b128_h64")
    tq, tk, tv = inputs.device_qkv((T, B, H, d), w["seed"], "bf16")
    lam = inputs.decay_schedule(H)
    tl = torch.from_numpy(lam).cuda()
    state = inputs.device_state((B, H, d, d), w["seed"] + 1)
    S = host(state).astype(np.float64)
    outs = torch.empty((T, B, H, d), dtype=torch.bfloat16, device="cuda")
    for t in range(T):
        la.lightning_attn_decode(tq[t], tk[t], tv[t], tl, state, out=outs[t])
    torch.cuda.synchronize()
    q, k, v = host(tq), host(tk), host(tv)
    o = host(outs)
    assert np.isfinite(o).all()
    num = den = 0.0
    for t in range(T):
        o_ref, _ = oracle.decode(q[t], k[t], v[t], lam, S)
        num = max(num, float(np.abs(o[t] - o_ref).max()))
        den = max(den, float(np.abs(o_ref).max()))
    eo = num / den
    es = whole_rel_err(state, S, dim=0, name="state")
    say("   err out %.3e state %.3e (all %d pairs, all %d steps)" % (eo, es, B * H, T))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("prefill_path", ["auto", "fused"], indirect=True)
def test_offsets_beyond_int32(prefill_path):
    """B=1 H=3 N=2^23+4099 d=128 bf16: every element of head 2 lies past
    2^31 elements (6.4 GB per tensor), so its loads, stores and state
    addresses need 64-bit offsets.  Decays 0.9, 0.999, 0.999: a token n rows
    back weighs at most 0.999^n, so an oracle run over a window of 2^17
    tokens before the compared rows, from a zero state, differs from the full
    recurrence by a factor 0.999^131072 < 1e-56 of the state: exact in double.
    Compared: head 2's first 4096 rows (no truncation), 1024 rows around the
    middle and the last 1024 rows with the final state; head 0's last rows."""
    torch = torch_mod()
    B, H, N, d = 1, 3, (1 << 23) + 4099, 128
    say("case offsets beyond int32 B=%d H=%d N=%d d=%d path=%s" % (B, H, N, d, prefill_path))
    assert 2 * N * d > 2 ** 31
    tq, tk, tv = inputs.device_qkv((B, H, N, d), 4242, "bf16")
    lam = np.array([0.9, 0.999, 0.999], np.float32)
    out = torch.full_like(tq, float("nan"))
    out, fin = la.lightning_attn_fwd(tq, tk, tv, torch.from_numpy(lam).cuda(), out=out)
    torch.cuda.synchronize()
    W = 1 << 17

    def window(h, a, b, cmp_from, want_state=False):
        q, k, v = (host(t[:, h:h + 1, a:b]) for t in (tq, tk, tv))
        o_ref, f_ref, _ = oracle.fwd(q, k, v, lam[h:h + 1])
        o = host(out[:, h:h + 1, cmp_from:b])
        assert np.isfinite(o).all()
        e = rel_err(o, o_ref[:, :, cmp_from - a:])
        es = rel_err(host(fin[:, h:h + 1]), f_ref) if want_state else 0.0
        say("   head %d rows [%d, %d) err out %.3e state %.3e" % (h, cmp_from, b, e, es))
        assert e <= TOL["bf16"] and es <= TOL["bf16"], (e, es)

    window(2, 0, 4096, 0)
    mid = N // 2
    window(2, mid - 512 - W, mid + 512, mid - 512)
    window(2, N - 1024 - W, N, N - 1024, want_state=True)
    window(0, N - 1024 - W, N, N - 1024, want_state=True)


@pytest.mark.parametrize("prefill_path", ["auto", "fused"], indirect=True)
def test_varlen_offsets_beyond_int32(prefill_path):
    """Packed [H, total, d] with H=3 and total = 2^23 + 4099 (head 2 past 2^31
    elements), five sequences, one of them empty, decays 0.9, 0.999, 0.999:
    per sequence, its first rows (exact) and its last 1024 rows from an
    oracle window of at most 2^17 tokens (see test_offsets_beyond_int32),
    and its final state."""
    torch = torch_mod()
    H, d = 3, 128
    cu = np.array([0, 1000, 3_000_000, 3_000_000, 6_500_017, (1 << 23) + 4099], np.int64)
    total = int(cu[-1])
    say("case varlen offsets beyond int32 H=%d total=%d seqs=%d path=%s"
        % (H, total, len(cu) - 1, prefill_path))
    tq, tk, tv = (t[0] for t in inputs.device_qkv((1, H, total, d), 4243, "bf16"))
    lam = np.array([0.9, 0.999, 0.999], np.float32)
    tcu = torch.from_numpy(cu.astype(np.int32)).cuda()
    out = torch.full_like(tq, float("nan"))
    out, fins = la.lightning_attn_fwd_varlen(tq, tk, tv, torch.from_numpy(lam).cuda(), tcu, out=out)
    torch.cuda.synchronize()
    W = 1 << 17
    for j in range(len(cu) - 1):
        s0, s1 = int(cu[j]), int(cu[j + 1])
        for h in (0, 2):
            if s1 == s0:
                e = rel_err(host(fins[j, h]), np.zeros((d, d)))
                say("   seq %d head %d empty: state err %.3e" % (j, h, e))
                assert e == 0.0
                continue
            spans = [(s0, min(s1, s0 + 2048), s0)]
            tail = max(s0, s1 - 1024)
            spans.append((max(s0, tail - W), s1, tail))
            for a, b, c in spans:
                q, k, v = (host(t[h:h + 1, a:b])[None] for t in (tq, tk, tv))
                o_ref, f_ref, _ = oracle.fwd(q, k, v, lam[h:h + 1])
                o = host(out[h:h + 1, c:b])[None]
                assert np.isfinite(o).all()
                e = rel_err(o, o_ref[:, :, c - a:])
                es = rel_err(host(fins[j, h]), f_ref[0, 0]) if b == s1 else 0.0
                say("   seq %d head %d rows [%d, %d) err out %.3e state %.3e" % (j, h, c, b, e, es))
                assert e <= TOL["bf16"] and es <= TOL["bf16"], (e, es)


def test_side_stream_and_concurrent_host_threads():
    """The library launches on the caller's current stream and keeps no
    per-call state: the same prefill issued on a side stream, and from two
    host threads at once (each on its own stream, with its own workspace),
    gives the default-stream result bit for bit."""
    import threading
    torch = torch_mod()
    B, H, N, d = 1, 8, 4096, 128
    say("case side stream and concurrent host threads")
    tq, tk, tv = inputs.device_qkv((B, H, N, d), 660, "bf16")
    lam = torch.from_numpy(inputs.decay_schedule(H)).cuda()
    ref_out, ref_fin = la.lightning_attn_fwd(tq, tk, tv, lam, segment_tokens=512)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        out, fin = la.lightning_attn_fwd(tq, tk, tv, lam, segment_tokens=512)
    side.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(fin, ref_fin)

    results, errors = {}, []

    def worker(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                res = []
                for _ in range(10):
                    res.append(la.lightning_attn_fwd(tq, tk, tv, lam, segment_tokens=512))
            st.synchronize()
            results[i] = res
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(2):
        for o, f in results[i]:
            assert torch.equal(o, ref_out) and torch.equal(f, ref_fin)


def test_misaligned_tensor_raises():
    """A contiguous view that starts 2 bytes past a 16-byte boundary is
    refused before any launch (LA_ERR_INVALID_ARG through the binding)."""
    torch = torch_mod()
    B, H, N, d = 1, 2, 256, 128
    n = B * H * N * d
    flat = torch.zeros(n + 8, dtype=torch.bfloat16, device="cuda")
    q = flat[1:n + 1].view(B, H, N, d)
    assert q.is_contiguous() and q.data_ptr() % 16 == 2
    k = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    lam = torch.full((H,), 0.9, device="cuda")
    with pytest.raises(la.LightningAttnError, match="LA_ERR_INVALID_ARG"):
        la.lightning_attn_fwd(q, k, k.clone(), lam)
