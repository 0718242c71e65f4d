"""GPU parity of the short-chunk kernel (block 16, 32, 64: 32- and 64-token
chunks, two workgroups per CU) and of the gated path (SiLU on q/k/v, per-head
RMS normalisation with a weight, sigmoid output gate) against the oracle.

Bar as everywhere: max |x - x_ref| / max |x_ref| over every element <= 2e-2
for bf16 inputs (the short-chunk kernel is the bf16, d = 128 path).
"""
import sys

import numpy as np
import pytest

import oracle
import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import inputs
from parity_util import ORACLE_CACHE, whole_rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2
LAMS = [0.9961, 0.3997, 2.0 ** -16, 1.0, 0.9]  # slow, fast, per-power branch, exactly 1


def torch_mod():
    import torch
    return torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    torch = torch_mod()
    return t.detach().to(torch.float32).cpu().numpy()


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.abs(b).max() if b.size else 0.0
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0)) if a.size else 0.0


def dev(x, bf16=True):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t.to(torch.bfloat16) if bf16 else t


# ------------------------------------------------------- short chunks


@pytest.mark.parametrize("block", [16, 32, 64])
@pytest.mark.parametrize("N,seg", [(1, 0), (33, 0), (64, 0), (65, 0), (300, 0), (1000, 256),
                                   (3000, 1024), (700, la.LA_SEGMENT_PER_SEQUENCE)])
def test_short_blocks_fixed(block, N, seg):
    """Fixed-length prefill on 32- or 64-token chunks: ragged tails, an
    initial state, segment cuts (local-state pass and scan), every decay
    branch."""
    torch = torch_mod()
    B, H, d = 2, len(LAMS), 128
    say("case short block=%d N=%d seg=%d" % (block, N, seg))
    q, k, v = inputs.host_qkv((B, H, N, d), 800 + N + block, dtype="bf16")
    lam = np.asarray(LAMS, np.float32)
    init = inputs.host_state((B, H, d, d), 801)
    out, fin = la.lightning_attn_fwd(dev(q), dev(k), dev(v), dev(lam, False), block=block,
                                     init_state=dev(init, False), segment_tokens=seg)
    torch.cuda.synchronize()
    o_ref, f_ref, _ = oracle.fwd(q, k, v, lam, init=init)
    ho = host(out)
    assert np.isfinite(ho).all()
    eo, ef = rel_err(ho, o_ref), rel_err(host(fin), f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL and ef <= TOL, (eo, ef)


@pytest.mark.parametrize("block", [32, 64])
@pytest.mark.parametrize("seg", [0, 200, la.LA_SEGMENT_PER_SEQUENCE])
@pytest.mark.parametrize("token_major", [False, True])
def test_short_blocks_varlen(block, seg, token_major):
    """Packed sequences (empty ones first, inside and last, one-token ones)
    on short chunks, both layouts."""
    torch = torch_mod()
    lens = [0, 300, 1, 0, 129, 64, 2000, 5, 0]
    H, d = len(LAMS), 128
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    q, k, v = inputs.host_qkv((H, total, d), 810 + block, dtype="bf16")
    lam = np.asarray(LAMS, np.float32)
    init = inputs.host_state((len(lens), H, d, d), 811)
    tq, tk, tv = dev(q), dev(k), dev(v)
    layout = la.LA_HEAD_MAJOR
    if token_major:
        tq, tk, tv = (t.transpose(0, 1).contiguous() for t in (tq, tk, tv))
        layout = la.LA_TOKEN_MAJOR
    out = torch.full_like(tq, float("nan"))
    out, fin = la.lightning_attn_fwd_varlen_layout(tq, tk, tv, dev(lam, False), dev(cu, False),
                                                   layout, block=block,
                                                   init_states=dev(init, False),
                                                   segment_tokens=seg, out=out)
    torch.cuda.synchronize()
    if token_major:
        out = out.transpose(0, 1)
    o_ref, f_ref, _ = oracle.fwd_varlen(q, k, v, lam, cu, init=init)
    ho = host(out)
    assert np.isfinite(ho).all()
    eo, ef = rel_err(ho, o_ref), rel_err(host(fin), f_ref)
    say("   varlen block=%d seg=%d tm=%s err out %.3e state %.3e" % (block, seg, token_major, eo,
                                                                     ef))
    assert eo <= TOL and ef <= TOL, (eo, ef)


def test_block_selects_the_kernel():
    """block 16 and 32 run the same 32-token kernel (bit-identical), 64 the
    64-token one and 128 the 128-token one (each within the bar, and 64 and
    128 not bit-identical: different chunkings round differently)."""
    torch = torch_mod()
    B, H, N, d = 1, 4, 2000, 128
    tq, tk, tv = inputs.device_qkv((B, H, N, d), 820, "bf16")
    lam = torch.from_numpy(inputs.decay_schedule(H)).cuda()
    res = {b: la.lightning_attn_fwd(tq, tk, tv, lam, block=b) for b in (16, 32, 64, 128, 256)}
    torch.cuda.synchronize()
    assert torch.equal(res[16][0], res[32][0]) and torch.equal(res[16][1], res[32][1])
    assert torch.equal(res[128][0], res[256][0])
    assert not torch.equal(res[64][0], res[128][0])
    assert not torch.equal(res[32][0], res[64][0])
    o_ref, f_ref, _ = oracle.fwd(host(tq), host(tk), host(tv), inputs.decay_schedule(H))
    for b, (o, f) in res.items():
        assert rel_err(host(o), o_ref) <= TOL and rel_err(host(f), f_ref) <= TOL, b


@pytest.mark.parametrize("N,level", [(20, 32), (50, 64), (64, 64), (300, 128)])
def test_block_auto_fixed(N, level):
    """LA_BLOCK_AUTO on a fixed-length call runs the level its length falls
    in (multi-level padding by input length): bit-identical to that level,
    and within the bar against the oracle."""
    torch = torch_mod()
    B, H, d = 3, len(LAMS), 128
    say("case block auto fixed N=%d level=%d" % (N, level))
    tq, tk, tv = inputs.device_qkv((B, H, N, d), 840 + N, "bf16")
    lam = torch.from_numpy(np.asarray(LAMS, np.float32)).cuda()
    init = dev(inputs.host_state((B, H, d, d), 841), False)
    oa, fa = la.lightning_attn_fwd(tq, tk, tv, lam, block=la.LA_BLOCK_AUTO, init_state=init)
    ol, fl = la.lightning_attn_fwd(tq, tk, tv, lam, block=level, init_state=init)
    torch.cuda.synchronize()
    assert torch.equal(oa, ol) and torch.equal(fa, fl)
    o_ref, f_ref, _ = oracle.fwd(host(tq), host(tk), host(tv), np.asarray(LAMS, np.float32),
                                 init=host(init))
    assert rel_err(host(oa), o_ref) <= TOL and rel_err(host(fa), f_ref) <= TOL


@pytest.mark.parametrize("lens,level", [([50, 50] + [1] * 18, 32), ([40] * 10 + [100] * 2, 64),
                                        ([2048, 2048] + [1] * 18, 128)])
def test_block_auto_varlen(lens, level):
    """LA_BLOCK_AUTO on packed batches (mean length = ceil(total / sequences)):
    the serving mix of 2 x 50 + 18 x 1 tokens takes block 32, a mean of 50
    takes 64, 2 x 2048 + 18 x 1 takes 128; bit-identical to that level with
    initial states and one segment per sequence, within the bar against the
    oracle."""
    torch = torch_mod()
    H, d = len(LAMS), 128
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    say("case block auto varlen total=%d seqs=%d level=%d" % (total, len(lens), level))
    q, k, v = inputs.host_qkv((H, total, d), 850 + level, dtype="bf16")
    lam = np.asarray(LAMS, np.float32)
    init = inputs.host_state((len(lens), H, d, d), 851)
    args = (dev(q), dev(k), dev(v), dev(lam, False), dev(cu, False))
    res = {}
    for b in (la.LA_BLOCK_AUTO, level):
        for seg in (0, la.LA_SEGMENT_PER_SEQUENCE):
            res[b, seg] = la.lightning_attn_fwd_varlen(*args, block=b,
                                                       init_states=dev(init, False),
                                                       segment_tokens=seg)
    torch.cuda.synchronize()
    o_ref, f_ref, _ = oracle.fwd_varlen(q, k, v, lam, cu, init=init)
    for seg in (0, la.LA_SEGMENT_PER_SEQUENCE):
        oa, fa = res[la.LA_BLOCK_AUTO, seg]
        ol, fl = res[level, seg]
        assert torch.equal(oa, ol) and torch.equal(fa, fl), seg
        assert rel_err(host(oa), o_ref) <= TOL and rel_err(host(fa), f_ref) <= TOL, seg


def test_short_deterministic():
    torch = torch_mod()
    tq, tk, tv = inputs.device_qkv((1, 8, 4096, 128), 830, "bf16")
    lam = torch.from_numpy(inputs.decay_schedule(8)).cuda()
    for block in (32, 64):
        o1, f1 = la.lightning_attn_fwd(tq, tk, tv, lam, block=block)
        o2, f2 = la.lightning_attn_fwd(tq, tk, tv, lam, block=block)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("block", [32, 64])
def test_short_full_layer_h64_n32k(block):
    """The 64-head 32768-token layer on short chunks: every output element
    and final-state entry against the oracle."""
    torch = torch_mod()
    w = inputs.WORKLOADS["layer_h64_n32k"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    say("case full layer_h64_n32k block=%d" % block)
    tq, tk, tv = inputs.device_qkv((B, H, N, d), w["seed"], "bf16")
    lam = inputs.decay_schedule(H)
    out, fin = la.lightning_attn_fwd(tq, tk, tv, torch.from_numpy(lam).cuda(), block=block)
    torch.cuda.synchronize()

    def compute():
        o_ref, f_ref, _ = oracle.fwd(host(tq), host(tk), host(tv), lam)
        return o_ref, f_ref

    o_ref, f_ref = ORACLE_CACHE.get("layer_h64_n32k", compute)
    del tq, tk, tv
    eo = whole_rel_err(out, o_ref, dim=1, name="out")
    ef = whole_rel_err(fin, f_ref, dim=1, name="final_state")
    say("   err out %.3e state %.3e (all %d heads)" % (eo, ef, H))
    assert eo <= TOL and ef <= TOL


# ------------------------------------------------ normalisation, SiLU, gate

ALL = la.LA_SILU_Q | la.LA_SILU_K | la.LA_SILU_V | la.LA_NORM | la.LA_GATE


def gated_inputs(shape, seed):
    q, k, v = inputs.host_qkv(shape, seed, dtype="bf16")
    g, _, _ = inputs.host_qkv(shape, seed + 1, dtype="bf16")
    g = inputs.round_to_bf16(g * np.float32(2.0 * np.sqrt(shape[-1])))  # gate inputs ~ N(0, 4)
    return q, k, v, g


def norm_weight(H, d, seed):
    rng = np.random.default_rng(seed)
    return rng.uniform(0.5, 1.5, (H, d)).astype(np.float32)


@pytest.mark.parametrize("flags", [0, la.LA_SILU_Q, la.LA_SILU_K, la.LA_SILU_V, la.LA_NORM,
                                   la.LA_GATE, la.LA_NORM | la.LA_GATE, ALL])
@pytest.mark.parametrize("seg", [0, 128])
def test_gated_flags(flags, seg):
    """Each part of the reading alone and all together, with and without
    segment cuts (the local-state pass applies the SiLU to K and V too), with
    a normalisation weight, against the oracle's gated reading."""
    torch = torch_mod()
    B, H, N, d = 2, len(LAMS), 700, 128
    say("case gated flags=%d seg=%d" % (flags, seg))
    q, k, v, g = gated_inputs((B, H, N, d), 840 + flags)
    lam = np.asarray(LAMS, np.float32)
    wgt = norm_weight(H, d, 841)
    init = inputs.host_state((B, H, d, d), 842)
    eps = 1e-5
    out, fin = la.lightning_attn_fwd_gated(dev(q), dev(k), dev(v), dev(lam, False), flags,
                                           gate=dev(g), norm_weight=dev(wgt, False), eps=eps,
                                           init_state=dev(init, False), segment_tokens=seg)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.fwd_gated(q, k, v, lam, flags, gate=g, weight=wgt, eps=eps, init=init)
    ho = host(out)
    assert np.isfinite(ho).all()
    eo, ef = rel_err(ho, o_ref), rel_err(host(fin), f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL and ef <= TOL, (eo, ef)


@pytest.mark.parametrize("seg", [200, la.LA_SEGMENT_PER_SEQUENCE])
@pytest.mark.parametrize("token_major", [False, True])
def test_gated_varlen(token_major, seg):
    """Packed sequences (empty ones included) with every part of the reading,
    against the oracle run on each sequence; segments cut inside sequences,
    or one segment per sequence."""
    torch = torch_mod()
    lens = [300, 0, 1, 129, 1024, 5, 0, 640]
    H, d = 3, 128
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    q, k, v, g = gated_inputs((H, total, d), 850)
    lam = inputs.decay_schedule(H)
    wgt = norm_weight(H, d, 851)
    init = inputs.host_state((len(lens), H, d, d), 852)
    tq, tk, tv, tg = dev(q), dev(k), dev(v), dev(g)
    layout = la.LA_HEAD_MAJOR
    if token_major:
        tq, tk, tv, tg = (t.transpose(0, 1).contiguous() for t in (tq, tk, tv, tg))
        layout = la.LA_TOKEN_MAJOR
    out, fin = la.lightning_attn_fwd_varlen_gated(tq, tk, tv, dev(lam, False), dev(cu, False),
                                                  ALL, gate=tg, norm_weight=dev(wgt, False),
                                                  layout=layout, init_states=dev(init, False),
                                                  segment_tokens=seg)
    torch.cuda.synchronize()
    if token_major:
        out = out.transpose(0, 1)
    ho, hf = host(out), host(fin)
    assert np.isfinite(ho).all()
    o_ref = np.zeros((H, total, d))
    f_ref = np.zeros((len(lens), H, d, d))
    for j in range(len(lens)):
        a, b = int(cu[j]), int(cu[j + 1])
        oj, fj = oracle.fwd_gated(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], lam, ALL,
                                  gate=g[None, :, a:b], weight=wgt, init=init[j][None])
        o_ref[:, a:b] = oj[0]
        f_ref[j] = fj[0]
    eo, ef = rel_err(ho, o_ref), rel_err(hf, f_ref)
    say("   err out %.3e state %.3e" % (eo, ef))
    assert eo <= TOL and ef <= TOL, (eo, ef)


@pytest.mark.parametrize("seg", [0, 256])
def test_gated_nothing_selected_is_the_plain_prefill(seg):
    """With no part selected the gated entry point runs the plain prefill:
    bit for bit lightning_attn_fwd at block 128."""
    torch = torch_mod()
    B, H, N, d = 1, len(LAMS), 1000, 128
    q, k, v, g = gated_inputs((B, H, N, d), 870)
    lam = np.asarray(LAMS, np.float32)
    init = inputs.host_state((B, H, d, d), 871)
    o1, f1 = la.lightning_attn_fwd_gated(dev(q), dev(k), dev(v), dev(lam, False), 0,
                                         init_state=dev(init, False), segment_tokens=seg)
    o2, f2 = la.lightning_attn_fwd(dev(q), dev(k), dev(v), dev(lam, False), block=128,
                                   init_state=dev(init, False), segment_tokens=seg)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_gated_rejects_bad_arguments():
    torch = torch_mod()
    B, H, N, d = 1, 2, 64, 128
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    lam = torch.full((H,), 0.9, device="cuda")
    with pytest.raises(la.LightningAttnError, match="LA_ERR_INVALID_ARG"):
        la.lightning_attn_fwd_gated(q, q, q, lam, 32)
    with pytest.raises(la.LightningAttnError, match="LA_ERR_INVALID_ARG"):
        la.lightning_attn_fwd_gated(q, q, q, lam, la.LA_NORM, eps=-1.0)
    with pytest.raises(ValueError):
        la.lightning_attn_fwd_gated(q, q, q, lam, la.LA_GATE)
    qf = torch.zeros(B, H, N, d, dtype=torch.float32, device="cuda")
    with pytest.raises(la.LightningAttnError, match="LA_ERR_UNSUPPORTED"):
        la.lightning_attn_fwd_gated(qf, qf, qf, lam, la.LA_NORM)
    q64 = torch.zeros(B, H, N, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(la.LightningAttnError, match="LA_ERR_UNSUPPORTED"):
        la.lightning_attn_fwd_gated(q64, q64, q64, lam, la.LA_NORM)


def test_gated_full_layer_h64_n32k():
    """Every part of the reading at the 64-head 32768-token layer shape: every
    output element against the oracle's gated reading."""
    torch = torch_mod()
    w = inputs.WORKLOADS["layer_h64_n32k"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    say("case full gated layer_h64_n32k")
    tq, tk, tv = inputs.device_qkv((B, H, N, d), w["seed"], "bf16")
    tg, _, _ = inputs.device_qkv((B, H, N, d), w["seed"] + 9, "bf16")
    tg = (tg.float() * (2.0 * np.sqrt(d))).to(torch.bfloat16)
    lam = inputs.decay_schedule(H)
    wgt = norm_weight(H, d, 861)
    out, fin = la.lightning_attn_fwd_gated(tq, tk, tv, torch.from_numpy(lam).cuda(), ALL, gate=tg,
                                           norm_weight=dev(wgt, False))
    torch.cuda.synchronize()
    ORACLE_CACHE.clear()
    o_ref, f_ref = oracle.fwd_gated(host(tq), host(tk), host(tv), lam, ALL, gate=host(tg),
                                    weight=wgt)
    del tq, tk, tv, tg
    eo = whole_rel_err(out, o_ref, dim=1, name="out")
    ef = whole_rel_err(fin, f_ref, dim=1, name="final_state")
    say("   err out %.3e state %.3e (all %d heads)" % (eo, ef, H))
    assert eo <= TOL and ef <= TOL
