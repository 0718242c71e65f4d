"""Double-precision CPU oracle for lightning attention -- TEST INFRASTRUCTURE.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
bench.py may import this package.  The product path never does.

Thin numpy/ctypes wrappers over oracle.c (see that file's header for what
each function computes and which passage of the MiniMax-01 report or the K3
reading notes it follows).  Inputs are float32 arrays holding the exact
values the GPU receives (bf16 widens to float32 exactly); results are
float64.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def load(path=None):
    """Loads (building first if absent) liboracle.so, or the library at path
    (or at $ORACLE_LIB, e.g. a sanitizer build of oracle.c)."""
    global _LIB
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _LIB is None and os.environ.get("ORACLE_LIB"):
        _LIB = _bind(ctypes.CDLL(os.environ["ORACLE_LIB"]))
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _LIB = _bind(ctypes.CDLL(_build.LIB))
    return _LIB


def _bind(lib):
    lib.oracle_default_threads.restype = _I
    lib.oracle_fwd_f64.argtypes = [_P, _P, _P, _P, _I, _I, _L, _I, _P, _P, _P, _I]
    lib.oracle_fwd_varlen_f64.argtypes = [_P, _P, _P, _P, _P, _I, _I, _L, _I, _P, _P, _P, _I]
    lib.oracle_fwd_varlen_snap_f64.argtypes = [_P, _P, _P, _P, _P, _I, _I, _L, _I, _P, _P, _P,
                                               _L, _P, _P, _I]
    lib.oracle_fwd_chdecay_f64.argtypes = [_P, _P, _P, _P, _I, _I, _L, _I, _P, _P, _P, _I]
    lib.oracle_fwd_gated_f64.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_double, _I, _I, _I, _L,
                                         _I, _P, _P, _P, _I]
    lib.oracle_bwd_f64.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _L, _I, _P, _P, _P, _P,
                                   _I]
    lib.oracle_decode_f64.argtypes = [_P, _P, _P, _P, _I, _I, _I, _P, _P, _I]
    lib.oracle_bruteforce_f64.argtypes = [_P, _P, _P, _P, _I, _I, _L, _I, _P, _P, _P, _I]
    lib.oracle_rows_f64.argtypes = [_P, _P, _P, ctypes.c_float, _I, _P, _L, _P, _P, _I]
    lib.oracle_state_entries_f64.argtypes = [_P, _P, ctypes.c_float, _I, _L, _P, _L, _P, _P, _I]
    for f in ("oracle_fwd_f64", "oracle_fwd_varlen_f64", "oracle_fwd_varlen_snap_f64",
              "oracle_bwd_f64", "oracle_fwd_chdecay_f64", "oracle_fwd_gated_f64",
              "oracle_decode_f64",
              "oracle_bruteforce_f64", "oracle_rows_f64", "oracle_state_entries_f64"):
        getattr(lib, f).restype = _I
    return lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def default_threads():
    return load().oracle_default_threads()


def fwd(q, k, v, decay, init=None, want_out=True, nthreads=0, lib=None):
    """Recurrence over q, k, v [B, H, N, d]; returns (out [B,H,N,d] or None,
    final_state [B,H,d,d], threads_used)."""
    lib = lib or load()
    q, k, v, decay = _f32(q), _f32(k), _f32(v), _f32(decay)
    B, H, N, d = q.shape
    init = _f64(init)
    out = np.empty((B, H, N, d), np.float64) if want_out else None
    fin = np.empty((B, H, d, d), np.float64)
    n = lib.oracle_fwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), B, H, N, d, _ptr(init),
                           _ptr(out), _ptr(fin), nthreads)
    return out, fin, n


def fwd_varlen(q, k, v, decay, cu_seqlens, init=None, want_out=True, nthreads=0, lib=None):
    """Packed recurrence over q, k, v [H, total, d]; the state restarts at
    every cu_seqlens boundary.  Returns (out, final_states [S,H,d,d], threads)."""
    lib = lib or load()
    q, k, v, decay = _f32(q), _f32(k), _f32(v), _f32(decay)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    H, total, d = q.shape
    S = cu.shape[0] - 1
    init = _f64(init)
    out = np.empty((H, total, d), np.float64) if want_out else None
    fin = np.empty((S, H, d, d), np.float64)
    n = lib.oracle_fwd_varlen_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(cu), S, H, total,
                                  d, _ptr(init), _ptr(out), _ptr(fin), nthreads)
    return out, fin, n


def fwd_varlen_snapshots(q, k, v, decay, cu_seqlens, interval, init=None, want_out=True,
                         nthreads=0, lib=None):
    """fwd_varlen that also returns the prefix states: snapshot m (from 1) of
    sequence j is the state after its first m * interval tokens, at row
    offsets[j] + m - 1, with offsets the exclusive prefix sum of
    floor(n_j / interval).  Returns (out, final_states, snapshots
    [rows, H, d, d], offsets [S + 1] int32)."""
    lib = lib or load()
    q, k, v, decay = _f32(q), _f32(k), _f32(v), _f32(decay)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    H, total, d = q.shape
    S = cu.shape[0] - 1
    assert interval >= 1
    offs = np.zeros(S + 1, np.int32)
    offs[1:] = np.cumsum(np.diff(cu.astype(np.int64)) // interval)
    init = _f64(init)
    out = np.empty((H, total, d), np.float64) if want_out else None
    fin = np.empty((S, H, d, d), np.float64)
    snaps = np.empty((int(offs[-1]), H, d, d), np.float64)
    lib.oracle_fwd_varlen_snap_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(cu), S, H, total,
                                   d, _ptr(init), _ptr(out), _ptr(fin), int(interval), _ptr(offs),
                                   _ptr(snaps), nthreads)
    return out, fin, snaps, offs


def fwd_chdecay(q, k, v, alpha, init=None, want_out=True, nthreads=0, lib=None):
    """Channel-wise decay: alpha [H, d] float32 (one decay per key channel of
    each head).  Returns (out [B,H,N,d] or None, final_state [B,H,d,d])."""
    lib = lib or load()
    q, k, v, alpha = _f32(q), _f32(k), _f32(v), _f32(alpha)
    B, H, N, d = q.shape
    assert alpha.shape == (H, d)
    init = _f64(init)
    out = np.empty((B, H, N, d), np.float64) if want_out else None
    fin = np.empty((B, H, d, d), np.float64)
    lib.oracle_fwd_chdecay_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), B, H, N, d, _ptr(init),
                               _ptr(out), _ptr(fin), nthreads)
    return out, fin


SILU_Q, SILU_K, SILU_V, NORM, GATE = 1, 2, 4, 8, 16


def fwd_gated(q, k, v, decay, flags, gate=None, weight=None, eps=1e-6, init=None, nthreads=0,
              lib=None):
    """The normalisation / SiLU / gate reading around the recurrence (see
    oracle.c): flags from SILU_Q, SILU_K, SILU_V, NORM, GATE; gate [B,H,N,d]
    (with GATE), weight [H, d] or None.  Returns (out [B,H,N,d], final_state
    [B,H,d,d])."""
    lib = lib or load()
    q, k, v, decay = _f32(q), _f32(k), _f32(v), _f32(decay)
    B, H, N, d = q.shape
    if flags & GATE:
        gate = _f32(gate)
        assert gate.shape == q.shape
    else:
        gate = None
    weight = None if weight is None else _f32(weight)
    init = _f64(init)
    out = np.empty((B, H, N, d), np.float64)
    fin = np.empty((B, H, d, d), np.float64)
    lib.oracle_fwd_gated_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(gate), _ptr(weight),
                             float(eps), int(flags), B, H, N, d, _ptr(init), _ptr(out), _ptr(fin),
                             nthreads)
    return out, fin


def bwd(q, k, v, decay, dout, dfin=None, init=None, nthreads=0, lib=None):
    """Gradients of fwd for q, k, v, dout [B, H, N, d]; dfin (gradient of the
    final state) and init [B, H, d, d] or None.  Returns (dq, dk, dv, dinit)
    in float64 (dinit [B, H, d, d])."""
    lib = lib or load()
    q, k, v, decay, dout = _f32(q), _f32(k), _f32(v), _f32(decay), _f32(dout)
    B, H, N, d = q.shape
    dfin, init = _f64(dfin), _f64(init)
    dq, dk, dv = (np.empty((B, H, N, d), np.float64) for _ in range(3))
    dinit = np.empty((B, H, d, d), np.float64)
    lib.oracle_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(dout), _ptr(dfin),
                       _ptr(init), B, H, N, d, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dinit),
                       nthreads)
    return dq, dk, dv, dinit


def decode(q, k, v, decay, state, nthreads=0, lib=None):
    """One recurrent step for q, k, v [B, H, d]; state [B, H, d, d] (float64)
    is updated in place.  Returns (out [B,H,d], threads)."""
    lib = lib or load()
    q, k, v, decay = _f32(q), _f32(k), _f32(v), _f32(decay)
    assert state.dtype == np.float64 and state.flags.c_contiguous
    B, H, d = q.shape
    out = np.empty((B, H, d), np.float64)
    n = lib.oracle_decode_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), B, H, d, _ptr(state),
                              _ptr(out), nthreads)
    return out, n


def bruteforce(q, k, v, decay, init=None, nthreads=0, lib=None):
    """Decayed left product, O(N^2 d) per head (small inputs only)."""
    lib = lib or load()
    q, k, v, decay = _f32(q), _f32(k), _f32(v), _f32(decay)
    B, H, N, d = q.shape
    init = _f64(init)
    out = np.empty((B, H, N, d), np.float64)
    fin = np.empty((B, H, d, d), np.float64)
    lib.oracle_bruteforce_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), B, H, N, d, _ptr(init),
                              _ptr(out), _ptr(fin), nthreads)
    return out, fin


def rows(q, k, v, decay, row_idx, init=None, nthreads=0, lib=None):
    """Selected output rows of ONE head: q, k, v [N, d] (rows up to max(row_idx)
    are read); decay is that head's float32 lambda.  Returns [len(rows), d]."""
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    d = q.shape[-1]
    r = np.ascontiguousarray(row_idx, dtype=np.int64)
    assert r.size == 0 or (r.min() >= 0 and r.max() < q.shape[0] and r.max() < k.shape[0])
    init = _f64(init)
    out = np.empty((r.size, d), np.float64)
    lib.oracle_rows_f64(_ptr(q), _ptr(k), _ptr(v), float(np.float32(decay)), d, _ptr(r), r.size,
                        _ptr(init), _ptr(out), nthreads)
    return out


def state_entries(k, v, decay, ij, init=None, nthreads=0, lib=None):
    """Entries (i, j) of ONE head's state after all N rows of k, v [N, d]."""
    lib = lib or load()
    k, v = _f32(k), _f32(v)
    N, d = k.shape
    ij = np.ascontiguousarray(ij, dtype=np.int32).reshape(-1, 2)
    assert ij.size == 0 or (ij.min() >= 0 and ij.max() < d)
    init = _f64(init)
    out = np.empty(ij.shape[0], np.float64)
    lib.oracle_state_entries_f64(_ptr(k), _ptr(v), float(np.float32(decay)), d, N, _ptr(ij),
                                 ij.shape[0], _ptr(init), _ptr(out), nthreads)
    return out
