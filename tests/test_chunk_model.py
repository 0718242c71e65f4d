"""A float64 numpy model of the blockwise decomposition the HIP kernels run,
checked against the oracle on the CPU.  Test-only; neither the oracle nor the
HIP path uses it.

What it models (MiniMax-01 report section 2.2.1, block expansion: left
product inside a block, right product between blocks, the block state
carried forward; section 3.2.2 LASP+: local prefix states, then a prefix
combination, then local outputs; K3 reading notes, CP for linear attention: a
sequence may be cut into chunks anywhere with identical results):

  * the per-head token space is the concatenation of all sequences; it is cut
    into equal segments of `seg` tokens, processed independently;
  * phase A: for each segment, the local state of its last piece (the part
    of the last sequence inside the segment), from zero, as one decayed sum;
  * phase B: a scan over segments that turns local states into the state
    entering every segment;
  * phase C: per segment, blocks of at most T tokens restarting at every
    sequence start:  O = a (.) (Q S) + ((Q K^T) (.) D) V,
    S <- lambda^L S + (b (.) K)^T V with a_r = lambda^(r+1),
    D_rc = lambda^(r-c) (r >= c), b_c = lambda^(L-1-c).
Optionally rounds to bf16 where the kernel does, to size the error budget.
"""
import numpy as np
import pytest

import oracle
from linear_attention_lightning_amd import inputs


def rel_err(a, b):
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0))


def bf(x, on):
    if not on:
        return x
    return inputs.round_to_bf16(np.asarray(x, np.float32)).astype(np.float64)


def seq_of(cu, tok):
    return int(np.searchsorted(cu, tok, side="right") - 1)


def piece_plan(ps, b, lam, C, R):
    """The local-state pass's cut of [ps, b): chunks of C tokens aligned to
    ps; those before the first one that can carry a nonzero float32 weight
    (lambda^n < 2^-160) are left out, and the rest is cut into 2^lg pieces,
    2^lg the power of two covering R times the weighted share (at most R).
    Returns the list of pieces [x0, x1)."""
    l2 = np.float32(np.log2(np.float32(lam)))
    tf = ps
    if l2 < 0:
        far = np.float32(b - ps) + np.float32(160.0) / l2
        if far >= np.float32(C):
            tf = ps + int(far / np.float32(C)) * C
    n = -(-(b - ps) // C)
    nw = -(-(b - tf) // C)
    want = -(-(nw * R) // n) if n > 0 else 1
    lg = 0
    while (1 << lg) < want and (1 << lg) < R:
        lg += 1
    out = []
    for r in range(1 << lg):
        x0 = tf + ((r * nw) >> lg) * C
        x1 = min(b, tf + (((r + 1) * nw) >> lg) * C)
        if x0 < x1:
            out.append((x0, x1))
    return out


def model(qh, kh, vh, lam, cu, T, seg, init=None, scan=True, bf16=False, pieces=None, C=64):
    """qh, kh, vh: [H, total, d] float64; cu: int64 [S+1]; init [S, H, d, d].
    pieces: None (phase A as one decayed sum), or R: phase A as the
    local-state pass runs it -- partial states of the pieces piece_plan cuts
    (chunks of C tokens), each weighted by lambda^(b - x1) in the scan.
    Returns (out [H, total, d], final [S, H, d, d])."""
    H, total, d = qh.shape
    S_n = len(cu) - 1
    init = np.zeros((S_n, H, d, d)) if init is None else init
    out = np.zeros_like(qh)
    fin = np.zeros((S_n, H, d, d))
    for j in range(S_n):
        if cu[j] == cu[j + 1]:
            fin[j] = init[j]
    nseg = -(-total // seg) if total else 0
    for h in range(H):
        L_ = float(lam[h])
        # phase A
        loc, gam = [], []
        for s in range(nseg):
            a, b = s * seg, min(total, (s + 1) * seg)
            jl = seq_of(cu, b - 1)
            ps = max(a, int(cu[jl]))
            if pieces is None:
                w = L_ ** (b - 1 - np.arange(ps, b))
                loc.append((kh[h, ps:b] * w[:, None]).T @ vh[h, ps:b])
            else:
                acc = np.zeros((d, d))
                for x0, x1 in piece_plan(ps, b, lam[h], C, pieces):
                    w = L_ ** (x1 - 1 - np.arange(x0, x1))
                    acc += L_ ** (b - x1) * ((kh[h, x0:x1] * w[:, None]).T @ vh[h, x0:x1])
                loc.append(acc)
            gam.append(L_ ** (b - ps))
        # phase B
        s_in = []
        carry = None
        for s in range(nseg):
            a, b = s * seg, min(total, (s + 1) * seg)
            jf = seq_of(cu, a)
            if not scan or cu[jf] == a:
                sin = init[jf, h]
            else:
                sin = carry
            s_in.append(sin)
            jl = seq_of(cu, b - 1)
            ps = max(a, int(cu[jl]))
            carry = gam[s] * (sin if ps == a else init[jl, h]) + loc[s]
        # phase C
        for s in range(nseg):
            a, b = s * seg, min(total, (s + 1) * seg)
            tok = a
            j = seq_of(cu, a)
            S = s_in[s].copy()
            while tok < b:
                pe = min(b, int(cu[j + 1]))
                for c0 in range(tok, pe, T):
                    c1 = min(c0 + T, pe)
                    L = c1 - c0
                    Q, K, V = qh[h, c0:c1], kh[h, c0:c1], vh[h, c0:c1]
                    r = np.arange(L)
                    av = L_ ** (r + 1)
                    D = np.where(r[:, None] >= r[None, :],
                                 L_ ** np.maximum(r[:, None] - r[None, :], 0), 0.0)
                    P = bf((Q @ K.T) * D, bf16)
                    O = av[:, None] * (Q @ bf(S, bf16)) + P @ V
                    out[h, c0:c1] = bf(O, bf16)
                    bv = L_ ** (L - 1 - r)
                    S = (L_ ** L) * S + bf(K * bv[:, None], bf16).T @ V
                if pe == cu[j + 1]:
                    fin[j, h] = S
                tok = pe
                if tok < b:
                    j = seq_of(cu, tok)
                    S = init[j, h].copy()
    return out, fin


def fixed_to_packed(x):
    B, H, N, d = x.shape
    return np.ascontiguousarray(x.transpose(1, 0, 2, 3).reshape(H, B * N, d)).astype(np.float64)


@pytest.mark.parametrize("B,H,N,d,T,seg,scan", [
    (1, 2, 256, 16, 128, 256, False),   # one segment per sequence, no scan
    (2, 2, 300, 8, 128, 300, False),    # tail block of 44 rows
    (1, 2, 1000, 8, 128, 256, True),    # 4 segments, ragged last
    (2, 3, 333, 8, 64, 128, True),      # segments straddle sequences
    (1, 1, 517, 4, 32, 96, True),       # segment not a multiple of the block
    (1, 2, 64, 8, 16, 16, True),        # one block per segment
])
def test_fixed_length_model_matches_oracle(B, H, N, d, T, seg, scan):
    q, k, v = inputs.host_qkv((B, H, N, d), 100 + N, dtype="fp32")
    lam = np.asarray([0.9961, 0.4, 0.75][:H], np.float32)
    init = inputs.host_state((B, H, d, d), 7).astype(np.float64)
    o, f, _ = oracle.fwd(q, k, v, lam, init=init)
    cu = np.arange(B + 1, dtype=np.int64) * N
    mo, mf = model(fixed_to_packed(q), fixed_to_packed(k), fixed_to_packed(v), lam, cu, T, seg,
                   init=init, scan=scan)
    assert rel_err(mo, fixed_to_packed(o)) < 1e-12
    assert rel_err(mf, f) < 1e-12


@pytest.mark.parametrize("T,seg", [(128, 256), (64, 192), (32, 32)])
def test_varlen_model_matches_oracle(T, seg):
    lens = [3, 0, 200, 129, 1, 0, 77, 256, 31]
    cu = inputs.cu_seqlens(lens).astype(np.int64)
    H, d = 2, 8
    q, k, v = inputs.host_qkv((H, int(cu[-1]), d), 5, dtype="fp32")
    lam = np.asarray([0.98, 0.5], np.float32)
    init = inputs.host_state((len(lens), H, d, d), 6).astype(np.float64)
    o, f, _ = oracle.fwd_varlen(q, k, v, lam, cu.astype(np.int32), init=init)
    mo, mf = model(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), lam, cu, T,
                   seg, init=init)
    assert rel_err(mo, o) < 1e-12
    assert rel_err(mf, f) < 1e-12


def test_bf16_rounding_budget_is_inside_tolerance():
    """With bf16 inputs and the kernel's roundings (S and P and b*K to bf16,
    output to bf16, fp32-range everything else) the error against the oracle
    stays far inside the 2e-2 bound (this sizes the error budget)."""
    B, H, N, d = 1, 2, 1024, 128
    q, k, v = inputs.host_qkv((B, H, N, d), 9, dtype="bf16")
    lam = np.asarray([0.9961, 0.3997], np.float32)
    o, f, _ = oracle.fwd(q, k, v, lam)
    cu = np.array([0, N], np.int64)
    mo, mf = model(fixed_to_packed(q), fixed_to_packed(k), fixed_to_packed(v), lam, cu, 128, 256,
                   bf16=True)
    eo, ef = rel_err(mo, fixed_to_packed(o)), rel_err(mf, f)
    assert eo < 2e-2 / 4 and ef < 2e-2 / 4, (eo, ef)


@pytest.mark.parametrize("R", [1, 2, 4, 16])
def test_local_state_pieces_model_matches_oracle(R):
    """Phase A computed as the local-state pass cuts it: the weighted part of
    each segment's last piece split into up to R pieces (fewer for the fast
    decays, whose leading chunks carry zero float32 weight and are left out),
    the partial states weighted by lambda^(b - x1) -- equal to the oracle."""
    lens = [700, 0, 1300, 64, 2000]
    cu = inputs.cu_seqlens(lens).astype(np.int64)
    H, d = 4, 8
    q, k, v = inputs.host_qkv((H, int(cu[-1]), d), 11, dtype="fp32")
    lam = np.asarray([0.999, 0.97, 0.6, 1.0], np.float32)
    init = inputs.host_state((len(lens), H, d, d), 12).astype(np.float64)
    o, f, _ = oracle.fwd_varlen(q, k, v, lam, cu.astype(np.int32), init=init)
    mo, mf = model(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), lam, cu, 32,
                   512, init=init, pieces=R, C=8)
    assert rel_err(mo, o) < 1e-12
    assert rel_err(mf, f) < 1e-12


def test_piece_plan_cuts():
    """A segment weighted throughout gets R pieces; a fast decay fewer (or
    one); no piece is empty or overlaps, and they end at the segment end."""
    full = piece_plan(0, 32768, 0.996, 64, 16)
    assert len(full) == 16 and full[-1][1] == 32768
    fast = piece_plan(0, 32768, 0.6065, 64, 16)
    assert len(fast) == 1 and fast[0][1] == 32768 and fast[0][0] > 32000
    mid = piece_plan(0, 32768, 0.98, 64, 16)
    assert 1 < len(mid) < 16
    for cut in (full, fast, mid):
        assert all(x0 < x1 for x0, x1 in cut)
        assert all(cut[i][1] == cut[i + 1][0] for i in range(len(cut) - 1))
