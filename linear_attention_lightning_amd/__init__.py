"""Lightning attention for AMD MI355X (gfx950): Python binding.

Thin ctypes layer over liblightning_attn.so (C ABI in include/lightning_attn.h).
It only checks tensors, allocates outputs and workspace with torch (device
memory and streams are all torch is used for) and passes raw pointers and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing or fails to load,
every call raises.

Entry points (same names as the C ABI):
  lightning_attn_fwd(q, k, v, decay, block=128, init_state=None, ...) -> (out, final_state)
  lightning_attn_fwd_timed(q, k, v, decay, phase_events, ...) -> (out, final_state)
  lightning_attn_fwd_noalloc(q, k, v, decay, ...) -> (out, final_state)   (no workspace)
  lightning_attn_fwd_gated(q, k, v, decay, flags, gate=None, norm_weight=None, eps=1e-6, ...)
      -> (out, final_state)   (SiLU on q/k/v, per-head RMS norm, sigmoid gate; LA_* flags)
  lightning_attn_fwd_varlen_gated(q, k, v, decay, cu_seqlens, flags, ...) -> (out, final_states)
  lightning_attn_fwd_layout(q, k, v, decay, layout, ...) -> (out, final_state)
  lightning_attn_fwd_varlen_layout(q, k, v, decay, cu_seqlens, layout, ...) -> (out, final_states)
  lightning_attn_fwd_varlen(q, k, v, decay, cu_seqlens, block=128, ...) -> (out, final_states)
  lightning_attn_fwd_varlen_snapshots(q, k, v, decay, cu_seqlens, snapshot_interval, ...)
      -> (out, final_states, snapshots, snapshot_offsets)
  lightning_attn_decode(q, k, v, decay, state, out=None) -> out   (state updated in place)
  lightning_attn_fwd_chdecay(q, k, v, alpha, ...) -> (out, final_state)   (alpha [H, d])
  lightning_attn_fwd_chdecay_varlen(q, k, v, alpha, cu_seqlens, ...) -> (out, final_states)
  lightning_attn_decode_chdecay(q, k, v, alpha, state, out=None) -> out
  lightning_attn_bwd(q, k, v, decay, dout, dfinal=None, init_state=None, ...)
      -> (dq, dk, dv, dinit)
  lightning_attn_bwd_varlen(q, k, v, decay, dout, cu_seqlens, ...) -> (dq, dk, dv, dinits)
  lightning_attn_fwd_save(q, k, v, decay, ...) -> (out, final_state, saved)
  lightning_attn_bwd_saved(q, k, v, decay, dout, saved, ...) -> (dq, dk, dv, dinit)
  lightning_attn_fwd_varlen_save(q, k, v, decay, cu_seqlens, ...) -> (out, final_states, saved)
  lightning_attn_bwd_varlen_saved(q, k, v, decay, dout, cu_seqlens, saved, ...)
      -> (dq, dk, dv, dinits)
  lightning_attn_mixed_step(decay, prefill_qkv, cu_seqlens, decode_qkv, decode_state, ...)
      -> (prefill_out, final_states, decode_out)   (decode_state updated in place)
"""
import ctypes
import os

__all__ = ["lightning_attn_fwd", "lightning_attn_fwd_timed", "lightning_attn_fwd_layout",
           "lightning_attn_fwd_noalloc", "lightning_attn_noalloc_scratch_bytes",
           "lightning_attn_fwd_gated", "lightning_attn_fwd_varlen_gated",
           "lightning_attn_fwd_gated_workspace_size",
           "lightning_attn_fwd_varlen_gated_workspace_size",
           "LA_SILU_Q", "LA_SILU_K", "LA_SILU_V", "LA_NORM", "LA_GATE",
           "lightning_attn_fwd_varlen", "lightning_attn_fwd_varlen_layout",
           "lightning_attn_fwd_varlen_snapshots", "snapshot_row_offsets", "lightning_attn_decode",
           "lightning_attn_mixed_step", "lightning_attn_bwd", "lightning_attn_bwd_workspace_size",
           "lightning_attn_fwd_chdecay", "lightning_attn_fwd_chdecay_workspace_size",
           "lightning_attn_decode_chdecay", "lightning_attn_bwd_varlen",
           "lightning_attn_bwd_varlen_workspace_size", "lightning_attn_saved_states_size",
           "lightning_attn_fwd_save", "lightning_attn_bwd_saved",
           "lightning_attn_varlen_saved_states_size", "lightning_attn_fwd_varlen_save",
           "lightning_attn_bwd_varlen_saved", "lightning_attn_fwd_chdecay_varlen",
           "lightning_attn_fwd_chdecay_varlen_workspace_size",
           "LA_HEAD_MAJOR", "LA_TOKEN_MAJOR", "LA_SEGMENT_PER_SEQUENCE", "LA_BLOCK_AUTO",
           "lightning_attn_fwd_workspace_size", "lightning_attn_fwd_varlen_workspace_size",
           "LightningAttnError", "load_library", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblightning_attn.so")

LA_FP32, LA_BF16 = 0, 1
LA_HEAD_MAJOR, LA_TOKEN_MAJOR = 0, 1  # la_layout
LA_SEGMENT_PER_SEQUENCE = -1          # segment_tokens: one segment per sequence
LA_BLOCK_AUTO = 0                     # block: level from the mean input length
LA_SILU_Q, LA_SILU_K, LA_SILU_V, LA_NORM, LA_GATE = 1, 2, 4, 8, 16  # gated-path flags
_STATUS = {0: "LA_OK", 1: "LA_ERR_INVALID_ARG", 2: "LA_ERR_UNSUPPORTED", 3: "LA_ERR_WORKSPACE",
           4: "LA_ERR_HIP"}

_lib = None


class LightningAttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        name = _STATUS.get(status, str(status))
        lib = load_library()
        msg = lib.lightning_attn_status_string(status).decode()
        if status == 4:
            msg += ": " + lib.lightning_attn_last_hip_error().decode()
        super().__init__("%s failed: %s (%s)" % (where, name, msg))


def load_library(path=None):
    """Loads liblightning_attn.so (built in-tree by
    `python -m linear_attention_lightning_amd.build`), or the build at
    `path` or at $LIGHTNING_ATTN_LIB (e.g. one with host-side sanitizers)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("LIGHTNING_ATTN_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("HIP library %s is not built; run "
                           "`python -m linear_attention_lightning_amd.build`" % p)
    # The library and PyTorch must use one HIP runtime (streams and device
    # pointers cross between them).  PyTorch ships its own libamdhip64 with
    # the same soname as the system one the library links, and the copy that
    # loads first serves both: importing torch first makes that PyTorch's.
    _torch()
    lib = ctypes.CDLL(p)
    P, I, L, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.lightning_attn_status_string.argtypes = [I]
    lib.lightning_attn_status_string.restype = ctypes.c_char_p
    lib.lightning_attn_version.restype = I
    lib.lightning_attn_last_hip_error.restype = ctypes.c_char_p
    lib.lightning_attn_fwd_workspace_size.argtypes = [I, I, L, I, I, I, L]
    lib.lightning_attn_fwd_workspace_size.restype = Z
    lib.lightning_attn_fwd.argtypes = [P, P, P, P, I, I, L, I, I, I, P, P, P, L, P, Z, P]
    lib.lightning_attn_fwd.restype = I
    lib.lightning_attn_fwd_timed.argtypes = [P, P, P, P, I, I, L, I, I, I, P, P, P, L, P, Z, P,
                                             ctypes.POINTER(P)]
    lib.lightning_attn_fwd_timed.restype = I
    lib.lightning_attn_fwd_gated_workspace_size.argtypes = [I, I, L, I, I, L]
    lib.lightning_attn_fwd_gated_workspace_size.restype = Z
    lib.lightning_attn_fwd_gated.argtypes = [P, P, P, P, I, I, L, I, I, I, I, P, P,
                                             ctypes.c_float, P, P, P, L, P, Z, P]
    lib.lightning_attn_fwd_gated.restype = I
    lib.lightning_attn_fwd_varlen_gated_workspace_size.argtypes = [I, I, L, I, I, L]
    lib.lightning_attn_fwd_varlen_gated_workspace_size.restype = Z
    lib.lightning_attn_fwd_varlen_gated.argtypes = [P, P, P, P, P, I, I, L, I, I, I, I, P, P,
                                                    ctypes.c_float, P, P, P, L, P, Z, P]
    lib.lightning_attn_fwd_varlen_gated.restype = I
    lib.lightning_attn_noalloc_scratch_bytes.argtypes = []
    lib.lightning_attn_noalloc_scratch_bytes.restype = Z
    lib.lightning_attn_fwd_noalloc.argtypes = [P, P, P, P, I, I, L, I, I, I, P, P, P, L, P]
    lib.lightning_attn_fwd_noalloc.restype = I
    lib.lightning_attn_fwd_layout.argtypes = [P, P, P, P, I, I, L, I, I, I, I, P, P, P, L, P, Z, P]
    lib.lightning_attn_fwd_layout.restype = I
    lib.lightning_attn_fwd_varlen_layout.argtypes = [P, P, P, P, P, I, I, L, I, I, I, I, P, P, P,
                                                     L, P, Z, P]
    lib.lightning_attn_fwd_varlen_layout.restype = I
    lib.lightning_attn_fwd_varlen_workspace_size.argtypes = [I, I, L, I, I, I, L]
    lib.lightning_attn_fwd_varlen_workspace_size.restype = Z
    lib.lightning_attn_fwd_varlen.argtypes = [P, P, P, P, P, I, I, L, I, I, I, P, P, P, L, P, Z, P]
    lib.lightning_attn_fwd_varlen.restype = I
    lib.lightning_attn_fwd_varlen_snapshots.argtypes = [P, P, P, P, P, I, I, L, I, I, I, I, P, P,
                                                        P, L, P, P, L, P, Z, P]
    lib.lightning_attn_fwd_varlen_snapshots.restype = I
    lib.lightning_attn_mixed_step.argtypes = [P, P, P, P, I, L, I, P, P, P, L, P, Z, P,
                                              P, P, P, P, P, I, P, P, I, I, I, I]
    lib.lightning_attn_mixed_step.restype = I
    lib.lightning_attn_fwd_chdecay_workspace_size.argtypes = [I, I, L, I, I, I, L]
    lib.lightning_attn_fwd_chdecay_workspace_size.restype = Z
    lib.lightning_attn_fwd_chdecay.argtypes = [P, P, P, P, I, I, L, I, I, I, I, P, P, P, L, P, Z,
                                               P]
    lib.lightning_attn_fwd_chdecay.restype = I
    lib.lightning_attn_fwd_chdecay_varlen_workspace_size.argtypes = [I, I, L, I, I, I, L]
    lib.lightning_attn_fwd_chdecay_varlen_workspace_size.restype = Z
    lib.lightning_attn_fwd_chdecay_varlen.argtypes = [P, P, P, P, P, I, I, L, I, I, I, I, P, P, P,
                                                      L, P, Z, P]
    lib.lightning_attn_fwd_chdecay_varlen.restype = I
    lib.lightning_attn_bwd_workspace_size.argtypes = [I, I, L, I, I, I, L]
    lib.lightning_attn_bwd_workspace_size.restype = Z
    lib.lightning_attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, L, I, I, I, I, L, P,
                                       Z, P]
    lib.lightning_attn_bwd.restype = I
    lib.lightning_attn_saved_states_size.argtypes = [I, I, L, I, I, I, L]
    lib.lightning_attn_saved_states_size.restype = Z
    lib.lightning_attn_fwd_save.argtypes = [P, P, P, P, I, I, L, I, I, I, I, P, P, P, L, P, Z, P, Z,
                                            P]
    lib.lightning_attn_fwd_save.restype = I
    lib.lightning_attn_bwd_saved.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, L, I, I, I, I,
                                             L, P, Z, P, Z, P]
    lib.lightning_attn_bwd_saved.restype = I
    lib.lightning_attn_varlen_saved_states_size.argtypes = [I, I, L, I, I, I, L]
    lib.lightning_attn_varlen_saved_states_size.restype = Z
    lib.lightning_attn_fwd_varlen_save.argtypes = [P, P, P, P, P, I, I, L, I, I, I, I, P, P, P, L,
                                                   P, Z, P, Z, P]
    lib.lightning_attn_fwd_varlen_save.restype = I
    lib.lightning_attn_bwd_varlen_saved.argtypes = [P, P, P, P, P, P, I, I, L, I, I, I, I, P, P,
                                                    P, P, P, P, L, P, Z, P, Z, P]
    lib.lightning_attn_bwd_varlen_saved.restype = I
    lib.lightning_attn_bwd_varlen_workspace_size.argtypes = [I, I, L, I, I, I, L]
    lib.lightning_attn_bwd_varlen_workspace_size.restype = Z
    lib.lightning_attn_bwd_varlen.argtypes = [P, P, P, P, P, P, I, I, L, I, I, I, I, P, P, P, P,
                                              P, P, L, P, Z, P]
    lib.lightning_attn_bwd_varlen.restype = I
    lib.lightning_attn_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, P]
    lib.lightning_attn_decode_chdecay.argtypes = [P, P, P, P, P, P, I, I, I, I, P]
    lib.lightning_attn_decode_chdecay.restype = I
    lib.lightning_attn_decode.restype = I
    if path is None:
        _lib = lib
    return lib


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_FP32
    raise TypeError("q, k, v must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device):
    if t.shape != shape:
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def lightning_attn_fwd_workspace_size(B, H, N, d, block=128, dtype=LA_BF16, segment_tokens=0):
    return load_library().lightning_attn_fwd_workspace_size(B, H, N, d, block, dtype,
                                                             segment_tokens)


def lightning_attn_fwd_varlen_workspace_size(num_seqs, H, total, d, block=128, dtype=LA_BF16,
                                             segment_tokens=0):
    return load_library().lightning_attn_fwd_varlen_workspace_size(num_seqs, H, total, d, block,
                                                                    dtype, segment_tokens)


def lightning_attn_fwd(q, k, v, decay, block=128, init_state=None, segment_tokens=0, out=None,
                       final_state=None, workspace=None):
    """Causal decayed linear attention over q, k, v [B, H, N, d] (bf16 or
    float32, contiguous, on one GPU).  decay: [H] float32.  Returns
    (out [B, H, N, d] in the input dtype, final_state [B, H, d, d] float32)."""
    return _fwd(q, k, v, decay, block, init_state, segment_tokens, out, final_state, workspace,
                None)


def lightning_attn_fwd_layout(q, k, v, decay, layout, block=128, init_state=None,
                              segment_tokens=0, out=None, final_state=None, workspace=None):
    """lightning_attn_fwd for either layout: q, k, v [B, H, N, d] for
    LA_HEAD_MAJOR, [B, N, H, d] for LA_TOKEN_MAJOR (a projection's output
    viewed per head, read in place).  out has q's layout; final_state is
    [B, H, d, d] float32 either way."""
    return _fwd(q, k, v, decay, block, init_state, segment_tokens, out, final_state, workspace,
                None, layout)


def lightning_attn_fwd_gated_workspace_size(B, H, N, d, dtype=LA_BF16, segment_tokens=0):
    return load_library().lightning_attn_fwd_gated_workspace_size(B, H, N, d, dtype,
                                                                   segment_tokens)


def lightning_attn_fwd_varlen_gated_workspace_size(num_seqs, H, total, d, dtype=LA_BF16,
                                                   segment_tokens=0):
    return load_library().lightning_attn_fwd_varlen_gated_workspace_size(num_seqs, H, total, d,
                                                                          dtype, segment_tokens)


def _gated_extras(q, flags, gate, norm_weight, H, d, dev):
    torch = _torch()
    if flags & LA_GATE:
        if gate is None:
            raise ValueError("LA_GATE needs a gate tensor")
        _check(gate, "gate", q.shape, q.dtype, dev)
    if norm_weight is not None:
        _check(norm_weight, "norm_weight", (H, d), torch.float32, dev)


def lightning_attn_fwd_gated(q, k, v, decay, flags, gate=None, norm_weight=None, eps=1e-6,
                             layout=LA_HEAD_MAJOR, init_state=None, segment_tokens=0, out=None,
                             final_state=None, workspace=None):
    """Prefill with the SiLU / normalisation / gate reading around the
    attention (see the C header): flags from LA_SILU_Q, LA_SILU_K, LA_SILU_V,
    LA_NORM, LA_GATE; gate like q (with LA_GATE); norm_weight [H, d] float32
    or None.  q, k, v [B, H, N, d] (LA_HEAD_MAJOR) or [B, N, H, d]
    (LA_TOKEN_MAJOR), bf16, d = 128.  Returns (out, final_state)."""
    torch = _torch()
    lib = load_library()
    if layout == LA_TOKEN_MAJOR:
        B, N, H, d = q.shape
    else:
        B, H, N, d = q.shape
    dev = q.device
    _check(k, "k", q.shape, q.dtype, dev)
    _check(v, "v", q.shape, q.dtype, dev)
    _check(q, "q", q.shape, q.dtype, dev)
    _check(decay, "decay", (H,), torch.float32, dev)
    _gated_extras(q, flags, gate, norm_weight, H, d, dev)
    if init_state is not None:
        _check(init_state, "init_state", (B, H, d, d), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", q.shape, q.dtype, dev)
    if final_state is None:
        final_state = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    _check(final_state, "final_state", (B, H, d, d), torch.float32, dev)
    dt = _dtype_code(q)
    ws_bytes = lib.lightning_attn_fwd_gated_workspace_size(B, H, N, d, dt, segment_tokens)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.lightning_attn_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), B, H, N, d, dt,
                                      layout, int(flags), _ptr(gate), _ptr(norm_weight),
                                      float(eps), _ptr(init_state), _ptr(out), _ptr(final_state),
                                      segment_tokens, _ptr(workspace), ws_have, _stream(dev))
    if st != 0:
        raise LightningAttnError(st, "lightning_attn_fwd_gated")
    return out, final_state


def lightning_attn_fwd_varlen_gated(q, k, v, decay, cu_seqlens, flags, gate=None,
                                    norm_weight=None, eps=1e-6, layout=LA_HEAD_MAJOR,
                                    init_states=None, segment_tokens=0, out=None,
                                    final_states=None, workspace=None):
    """Packed form of lightning_attn_fwd_gated: q, k, v [H, total, d]
    (LA_HEAD_MAJOR) or [total, H, d] (LA_TOKEN_MAJOR); gate like q.  Returns
    (out, final_states [num_seqs, H, d, d])."""
    torch = _torch()
    lib = load_library()
    if layout == LA_TOKEN_MAJOR:
        total, H, d = q.shape
    else:
        H, total, d = q.shape
    dev = q.device
    _check(k, "k", q.shape, q.dtype, dev)
    _check(v, "v", q.shape, q.dtype, dev)
    _check(q, "q", q.shape, q.dtype, dev)
    _check(decay, "decay", (H,), torch.float32, dev)
    _gated_extras(q, flags, gate, norm_weight, H, d, dev)
    S = cu_seqlens.numel() - 1
    _check(cu_seqlens, "cu_seqlens", (S + 1,), torch.int32, dev)
    if init_states is not None:
        _check(init_states, "init_states", (S, H, d, d), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", q.shape, q.dtype, dev)
    if final_states is None:
        final_states = torch.empty((S, H, d, d), dtype=torch.float32, device=dev)
    _check(final_states, "final_states", (S, H, d, d), torch.float32, dev)
    dt = _dtype_code(q)
    ws_bytes = lib.lightning_attn_fwd_varlen_gated_workspace_size(S, H, total, d, dt,
                                                                  segment_tokens)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.lightning_attn_fwd_varlen_gated(
        _ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(cu_seqlens), S, H, total, d, dt, layout,
        int(flags), _ptr(gate), _ptr(norm_weight), float(eps), _ptr(init_states), _ptr(out),
        _ptr(final_states), segment_tokens, _ptr(workspace), ws_have, _stream(dev))
    if st != 0:
        raise LightningAttnError(st, "lightning_attn_fwd_varlen_gated")
    return out, final_states


def lightning_attn_noalloc_scratch_bytes():
    """Bytes of the library's own per-GPU scratch array, which
    lightning_attn_fwd_noalloc uses in place of a workspace."""
    return load_library().lightning_attn_noalloc_scratch_bytes()


def lightning_attn_fwd_noalloc(q, k, v, decay, block=128, init_state=None, segment_tokens=0,
                               out=None, final_state=None):
    """lightning_attn_fwd without a workspace: the library keeps the
    prefill's scratch in its own device array (see the C header for the
    limit and for calls that overlap on one GPU).  The C call allocates
    nothing; pass `out` and `final_state` to allocate nothing here either."""
    torch = _torch()
    lib = load_library()
    B, H, N, d = q.shape
    dev = q.device
    _check(k, "k", q.shape, q.dtype, dev)
    _check(v, "v", q.shape, q.dtype, dev)
    _check(q, "q", q.shape, q.dtype, dev)
    _check(decay, "decay", (H,), torch.float32, dev)
    if init_state is not None:
        _check(init_state, "init_state", (B, H, d, d), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", q.shape, q.dtype, dev)
    if final_state is None:
        final_state = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    _check(final_state, "final_state", (B, H, d, d), torch.float32, dev)
    st = lib.lightning_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), B, H, N, d, block,
                                        _dtype_code(q), _ptr(init_state), _ptr(out),
                                        _ptr(final_state), segment_tokens, _stream(dev))
    if st != 0:
        raise LightningAttnError(st, "lightning_attn_fwd_noalloc")
    return out, final_state


def lightning_attn_fwd_timed(q, k, v, decay, phase_events, block=128, init_state=None,
                             segment_tokens=0, out=None, final_state=None, workspace=None):
    """lightning_attn_fwd that also records 4 caller-owned HIP events on the
    current stream: before the first launch, after the local-state pass,
    after the segment scan and after the output pass.  phase_events: 4 raw
    hipEvent_t handles (for example torch.cuda.Event(...).cuda_event of
    events recorded once beforehand, so that the handles exist)."""
    if len(phase_events) != 4 or not all(phase_events):
        raise ValueError("phase_events must hold 4 created hipEvent_t handles")
    return _fwd(q, k, v, decay, block, init_state, segment_tokens, out, final_state, workspace,
                phase_events)


def _fwd(q, k, v, decay, block, init_state, segment_tokens, out, final_state, workspace,
         phase_events, layout=None):
    torch = _torch()
    lib = load_library()
    if layout == LA_TOKEN_MAJOR:
        B, N, H, d = q.shape
    elif layout in (None, LA_HEAD_MAJOR):
        B, H, N, d = q.shape
    else:
        raise ValueError("layout must be LA_HEAD_MAJOR or LA_TOKEN_MAJOR")
    dev = q.device
    _check(k, "k", q.shape, q.dtype, dev)
    _check(v, "v", q.shape, q.dtype, dev)
    _check(q, "q", q.shape, q.dtype, dev)
    _check(decay, "decay", (H,), torch.float32, dev)
    if init_state is not None:
        _check(init_state, "init_state", (B, H, d, d), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", q.shape, q.dtype, dev)
    if final_state is None:
        final_state = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    _check(final_state, "final_state", (B, H, d, d), torch.float32, dev)
    dt = _dtype_code(q)
    ws_bytes = lib.lightning_attn_fwd_workspace_size(B, H, N, d, block, dt, segment_tokens)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(decay), B, H, N, d, block, dt, _ptr(init_state),
            _ptr(out), _ptr(final_state), segment_tokens, _ptr(workspace), ws_have, _stream(dev))
    if layout is not None:
        st = lib.lightning_attn_fwd_layout(*args[:10], layout, *args[10:])
        name = "lightning_attn_fwd_layout"
    elif phase_events is None:
        st = lib.lightning_attn_fwd(*args)
        name = "lightning_attn_fwd"
    else:
        ev = (ctypes.c_void_p * 4)(*[int(e) for e in phase_events])
        st = lib.lightning_attn_fwd_timed(*args, ev)
        name = "lightning_attn_fwd_timed"
    if st != 0:
        raise LightningAttnError(st, name)
    return out, final_state


def lightning_attn_fwd_varlen(q, k, v, decay, cu_seqlens, block=128, init_states=None,
                              segment_tokens=0, out=None, final_states=None, workspace=None):
    """Packed variable-length form: q, k, v [H, total, d]; cu_seqlens int32
    [num_seqs + 1] on the same device (0 first, total last, non-decreasing).
    Returns (out [H, total, d], final_states [num_seqs, H, d, d] float32)."""
    return _fwd_varlen(q, k, v, decay, cu_seqlens, block, init_states, segment_tokens, out,
                       final_states, workspace, None)


def lightning_attn_fwd_varlen_layout(q, k, v, decay, cu_seqlens, layout, block=128,
                                     init_states=None, segment_tokens=0, out=None,
                                     final_states=None, workspace=None):
    """lightning_attn_fwd_varlen for either layout: q, k, v [H, total, d] for
    LA_HEAD_MAJOR, [total, H, d] for LA_TOKEN_MAJOR."""
    return _fwd_varlen(q, k, v, decay, cu_seqlens, block, init_states, segment_tokens, out,
                       final_states, workspace, layout)


def snapshot_row_offsets(cu_seqlens, snapshot_interval):
    """Row offsets of each sequence's prefix-state snapshots in the packed
    snapshot buffer: the exclusive prefix sum of floor(n_j / interval), as a
    list of num_seqs + 1 Python ints (the last one is the row count)."""
    if snapshot_interval < 1:
        raise ValueError("snapshot_interval must be >= 1")
    cu = [int(x) for x in cu_seqlens.tolist()]
    offs = [0]
    for j in range(len(cu) - 1):
        offs.append(offs[-1] + (cu[j + 1] - cu[j]) // snapshot_interval)
    return offs


def lightning_attn_fwd_varlen_snapshots(q, k, v, decay, cu_seqlens, snapshot_interval,
                                        layout=LA_HEAD_MAJOR, block=128, init_states=None,
                                        segment_tokens=0, out=None, final_states=None,
                                        snapshots=None, snapshot_offsets=None, workspace=None):
    """lightning_attn_fwd_varlen_layout that also stores the state of every
    sequence after each multiple of snapshot_interval of its tokens (a prefix
    cache).  snapshot_offsets: int32 [num_seqs + 1] on the device (default:
    the exclusive prefix sum of floor(n_j / interval), computed from
    cu_seqlens on the host); snapshot m (from 1) of sequence j is row
    snapshot_offsets[j] + m - 1 of snapshots [rows, H, d, d] float32.
    Returns (out, final_states, snapshots, snapshot_offsets)."""
    torch = _torch()
    dev = q.device
    if snapshot_offsets is None:
        offs = snapshot_row_offsets(cu_seqlens, snapshot_interval)
        snapshot_offsets = torch.tensor(offs, dtype=torch.int32, device=dev)
        rows = offs[-1]
    else:
        rows = None
    H = q.shape[1] if layout == LA_TOKEN_MAJOR else q.shape[0]
    d = q.shape[2]
    if snapshots is None:
        if rows is None:
            rows = int(snapshot_offsets[-1].item())
        snapshots = torch.empty((rows, H, d, d), dtype=torch.float32, device=dev)
    if snapshots.dim() != 4 or snapshots.shape[1:] != (H, d, d):
        raise ValueError("snapshots must be [rows, H, d, d]")
    _check(snapshots, "snapshots", snapshots.shape, torch.float32, dev)
    _check(snapshot_offsets, "snapshot_offsets", (cu_seqlens.numel(),), torch.int32, dev)
    iv = snapshot_interval
    if snapshots.numel() == 0:
        # no snapshot is due: an interval beyond every sequence stores none
        iv = max(int(q.shape[0] if layout == LA_TOKEN_MAJOR else q.shape[1]), 0) + 1
    out, final_states = _fwd_varlen(q, k, v, decay, cu_seqlens, block, init_states,
                                    segment_tokens, out, final_states, workspace, layout,
                                    (iv, snapshot_offsets, snapshots))
    return out, final_states, snapshots, snapshot_offsets


def _fwd_varlen(q, k, v, decay, cu_seqlens, block, init_states, segment_tokens, out,
                final_states, workspace, layout, snap=None):
    torch = _torch()
    lib = load_library()
    if layout == LA_TOKEN_MAJOR:
        total, H, d = q.shape
    elif layout in (None, LA_HEAD_MAJOR):
        H, total, d = q.shape
    else:
        raise ValueError("layout must be LA_HEAD_MAJOR or LA_TOKEN_MAJOR")
    dev = q.device
    _check(k, "k", q.shape, q.dtype, dev)
    _check(v, "v", q.shape, q.dtype, dev)
    _check(q, "q", q.shape, q.dtype, dev)
    _check(decay, "decay", (H,), torch.float32, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of num_seqs + 1 offsets")
    S = cu_seqlens.numel() - 1
    _check(cu_seqlens, "cu_seqlens", (S + 1,), torch.int32, dev)
    if init_states is not None:
        _check(init_states, "init_states", (S, H, d, d), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", q.shape, q.dtype, dev)
    if final_states is None:
        final_states = torch.empty((S, H, d, d), dtype=torch.float32, device=dev)
    _check(final_states, "final_states", (S, H, d, d), torch.float32, dev)
    dt = _dtype_code(q)
    ws_bytes = lib.lightning_attn_fwd_varlen_workspace_size(S, H, total, d, block, dt,
                                                            segment_tokens)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = workspace.numel() * workspace.element_size() if workspace is not None else 0
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(cu_seqlens), S, H, total, d, block, dt)
    tail = (_ptr(init_states), _ptr(out), _ptr(final_states), segment_tokens, _ptr(workspace),
            ws_have, _stream(dev))
    if snap is not None:
        iv, offs, rows = snap
        st = lib.lightning_attn_fwd_varlen_snapshots(*head, layout, *tail[:3], iv, _ptr(offs),
                                                     _ptr(rows), *tail[3:])
        name = "lightning_attn_fwd_varlen_snapshots"
    elif layout is None:
        st = lib.lightning_attn_fwd_varlen(*head, *tail)
        name = "lightning_attn_fwd_varlen"
    else:
        st = lib.lightning_attn_fwd_varlen_layout(*head, layout, *tail)
        name = "lightning_attn_fwd_varlen_layout"
    if st != 0:
        raise LightningAttnError(st, name)
    return out, final_states


def lightning_attn_decode_chdecay(q, k, v, alpha, state, out=None):
    """One decode step with channel-wise decay: alpha [H, d] float32; state
    [B, H, d, d] float32 is updated in place (row i decays by alpha[h][i])."""
    return _decode(q, k, v, alpha, state, out, channelwise=True)


def lightning_attn_decode(q, k, v, decay, state, out=None):
    """One decode step: q, k, v [B, H, d]; state [B, H, d, d] float32 is
    updated in place (state <- lambda state + k^T v); returns out = q state."""
    return _decode(q, k, v, decay, state, out, channelwise=False)


def _decode(q, k, v, decay, state, out, channelwise):
    torch = _torch()
    lib = load_library()
    B, H, d = q.shape
    dev = q.device
    _check(k, "k", q.shape, q.dtype, dev)
    _check(v, "v", q.shape, q.dtype, dev)
    _check(q, "q", q.shape, q.dtype, dev)
    _check(decay, "alpha" if channelwise else "decay", (H, d) if channelwise else (H,),
           torch.float32, dev)
    _check(state, "state", (B, H, d, d), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", q.shape, q.dtype, dev)
    fn = lib.lightning_attn_decode_chdecay if channelwise else lib.lightning_attn_decode
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(state), _ptr(out), B, H, d,
            _dtype_code(q), _stream(dev))
    if st != 0:
        raise LightningAttnError(st, "lightning_attn_decode_chdecay" if channelwise
                                 else "lightning_attn_decode")
    return out


def lightning_attn_mixed_step(decay, prefill_qkv, cu_seqlens, decode_qkv, decode_state,
                              layout=LA_HEAD_MAJOR, block=128, init_states=None,
                              segment_tokens=0, prefill_out=None, final_states=None,
                              decode_out=None, workspace=None, prefill_stream=None,
                              decode_stream=None):
    """One mixed serving step: packed prefill of the sequences with several
    new tokens (prefill_qkv: q, k, v [H, total, d], or [total, H, d] for
    LA_TOKEN_MAJOR; cu_seqlens int32 [num_seqs + 1]) on prefill_stream, and
    one decode step of decode_B single-token sequences (decode_qkv: q, k, v
    [decode_B, H, d]; decode_state [decode_B, H, d, d] float32, updated in
    place) on decode_stream, launched back to back so that they run
    concurrently.  Streams are torch.cuda.Stream objects (default: the
    current stream).  Returns (prefill_out, final_states, decode_out); the
    caller waits on both streams before using them."""
    torch = _torch()
    lib = load_library()
    pq, pk, pv = prefill_qkv
    dq, dk, dv = decode_qkv
    if layout == LA_TOKEN_MAJOR:
        total, H, d = pq.shape
    elif layout == LA_HEAD_MAJOR:
        H, total, d = pq.shape
    else:
        raise ValueError("layout must be LA_HEAD_MAJOR or LA_TOKEN_MAJOR")
    dev = pq.device
    for t, n in ((pk, "prefill k"), (pv, "prefill v"), (pq, "prefill q")):
        _check(t, n, pq.shape, pq.dtype, dev)
    _check(decay, "decay", (H,), torch.float32, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of num_seqs + 1 offsets")
    S = cu_seqlens.numel() - 1
    _check(cu_seqlens, "cu_seqlens", (S + 1,), torch.int32, dev)
    B = dq.shape[0]
    for t, n in ((dk, "decode k"), (dv, "decode v"), (dq, "decode q")):
        _check(t, n, (B, H, d), pq.dtype, dev)
    _check(decode_state, "decode_state", (B, H, d, d), torch.float32, dev)
    if init_states is not None:
        _check(init_states, "init_states", (S, H, d, d), torch.float32, dev)
    cur = torch.cuda.current_stream(dev)
    ps = prefill_stream or cur
    ds = decode_stream or cur
    if prefill_out is None:
        prefill_out = torch.empty_like(pq)
    if final_states is None:
        final_states = torch.empty((S, H, d, d), dtype=torch.float32, device=dev)
    if decode_out is None:
        decode_out = torch.empty_like(dq)
    _check(prefill_out, "prefill_out", pq.shape, pq.dtype, dev)
    _check(final_states, "final_states", (S, H, d, d), torch.float32, dev)
    _check(decode_out, "decode_out", dq.shape, dq.dtype, dev)
    dt = _dtype_code(pq)
    ws_bytes = lib.lightning_attn_fwd_varlen_workspace_size(S, H, total, d, block, dt,
                                                            segment_tokens)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = workspace.numel() * workspace.element_size() if workspace is not None else 0
    # tensors made here on the current stream and used on another one
    for t, s_ in ((prefill_out, ps), (final_states, ps), (workspace, ps), (decode_out, ds)):
        if t is not None and s_ != cur:
            t.record_stream(s_)
    st = lib.lightning_attn_mixed_step(
        _ptr(pq), _ptr(pk), _ptr(pv), _ptr(cu_seqlens), S, total, layout, _ptr(init_states),
        _ptr(prefill_out), _ptr(final_states), segment_tokens, _ptr(workspace), ws_have,
        ctypes.c_void_p(ps.cuda_stream), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(decode_state),
        _ptr(decode_out), B, ctypes.c_void_p(ds.cuda_stream), _ptr(decay), H, d, block, dt)
    if st != 0:
        raise LightningAttnError(st, "lightning_attn_mixed_step")
    return prefill_out, final_states, decode_out


def lightning_attn_bwd_workspace_size(B, H, N, d, block=128, dtype=LA_BF16, segment_tokens=0):
    return load_library().lightning_attn_bwd_workspace_size(B, H, N, d, block, dtype,
                                                             segment_tokens)


def lightning_attn_bwd(q, k, v, decay, dout, dfinal=None, init_state=None, layout=LA_HEAD_MAJOR,
                       block=128, segment_tokens=0, want_dinit=True, dq=None, dk=None, dv=None,
                       dinit=None, workspace=None):
    """Gradients of lightning_attn_fwd_layout: q, k, v, dout [B, H, N, d]
    (LA_HEAD_MAJOR) or [B, N, H, d] (LA_TOKEN_MAJOR); dfinal (gradient of the
    final state) and init_state [B, H, d, d] float32 or None.  Returns
    (dq, dk, dv, dinit) -- dinit [B, H, d, d] float32, or None when
    want_dinit is false."""
    return _bwd_fixed(q, k, v, decay, dout, dfinal, init_state, layout, block, segment_tokens,
                      want_dinit, dq, dk, dv, dinit, workspace, False, None)


def lightning_attn_bwd_saved(q, k, v, decay, dout, saved, dfinal=None, init_state=None,
                             layout=LA_HEAD_MAJOR, block=128, segment_tokens=0, want_dinit=True,
                             dq=None, dk=None, dv=None, dinit=None, workspace=None):
    """lightning_attn_bwd with the segment states `saved` kept by
    lightning_attn_fwd_save on the same inputs and arguments (None when
    lightning_attn_saved_states_size is 0)."""
    return _bwd_fixed(q, k, v, decay, dout, dfinal, init_state, layout, block, segment_tokens,
                      want_dinit, dq, dk, dv, dinit, workspace, True, saved)


def lightning_attn_saved_states_size(B, H, N, d, block=128, dtype=LA_BF16, segment_tokens=0):
    return load_library().lightning_attn_saved_states_size(B, H, N, d, block, dtype,
                                                            segment_tokens)


def lightning_attn_fwd_save(q, k, v, decay, layout=LA_HEAD_MAJOR, block=128, init_state=None,
                            segment_tokens=0, out=None, final_state=None, saved=None,
                            workspace=None):
    """The forward of a training pair: lightning_attn_fwd_layout that also
    keeps, for lightning_attn_bwd_saved, the transposed state entering every
    segment of the backward's plan.  Returns (out, final_state, saved) --
    saved a float32 device tensor, or None when nothing needs keeping.  The
    workspace is sized by lightning_attn_bwd_workspace_size."""
    torch = _torch()
    lib = load_library()
    if layout == LA_TOKEN_MAJOR:
        B, N, H, d = q.shape
    elif layout == LA_HEAD_MAJOR:
        B, H, N, d = q.shape
    else:
        raise ValueError("layout must be LA_HEAD_MAJOR or LA_TOKEN_MAJOR")
    dev = q.device
    for t, n in ((k, "k"), (v, "v"), (q, "q")):
        _check(t, n, q.shape, q.dtype, dev)
    _check(decay, "decay", (H,), torch.float32, dev)
    if init_state is not None:
        _check(init_state, "init_state", (B, H, d, d), torch.float32, dev)
    out = torch.empty_like(q) if out is None else out
    _check(out, "out", q.shape, q.dtype, dev)
    if final_state is None:
        final_state = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    _check(final_state, "final_state", (B, H, d, d), torch.float32, dev)
    dt = _dtype_code(q)
    sv_bytes = lib.lightning_attn_saved_states_size(B, H, N, d, block, dt, segment_tokens)
    if saved is None and sv_bytes:
        saved = torch.empty(sv_bytes // 4, dtype=torch.float32, device=dev)
    sv_have = saved.numel() * saved.element_size() if saved is not None else 0
    ws_bytes = lib.lightning_attn_bwd_workspace_size(B, H, N, d, block, dt, segment_tokens)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.lightning_attn_fwd_save(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), B, H, N, d, block, dt,
                                     layout, _ptr(init_state), _ptr(out), _ptr(final_state),
                                     segment_tokens, _ptr(saved), sv_have, _ptr(workspace),
                                     ws_have, _stream(dev))
    if st != 0:
        raise LightningAttnError(st, "lightning_attn_fwd_save")
    return out, final_state, saved


def _bwd_fixed(q, k, v, decay, dout, dfinal, init_state, layout, block, segment_tokens,
               want_dinit, dq, dk, dv, dinit, workspace, with_saved, saved):
    torch = _torch()
    lib = load_library()
    if layout == LA_TOKEN_MAJOR:
        B, N, H, d = q.shape
    elif layout == LA_HEAD_MAJOR:
        B, H, N, d = q.shape
    else:
        raise ValueError("layout must be LA_HEAD_MAJOR or LA_TOKEN_MAJOR")
    dev = q.device
    for t, n in ((k, "k"), (v, "v"), (dout, "dout"), (q, "q")):
        _check(t, n, q.shape, q.dtype, dev)
    _check(decay, "decay", (H,), torch.float32, dev)
    for t, n in ((dfinal, "dfinal"), (init_state, "init_state")):
        if t is not None:
            _check(t, n, (B, H, d, d), torch.float32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, n, q.shape, q.dtype, dev)
    if want_dinit and dinit is None:
        dinit = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    if dinit is not None:
        _check(dinit, "dinit", (B, H, d, d), torch.float32, dev)
    dt = _dtype_code(q)
    ws_bytes = lib.lightning_attn_bwd_workspace_size(B, H, N, d, block, dt, segment_tokens)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if with_saved:
        if saved is not None:
            _check(saved, "saved", saved.shape, torch.float32, dev)
        sv_have = saved.numel() * saved.element_size() if saved is not None else 0
        st = lib.lightning_attn_bwd_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(dout),
                                          _ptr(dfinal), _ptr(init_state), _ptr(dq), _ptr(dk),
                                          _ptr(dv), _ptr(dinit), B, H, N, d, block, dt, layout,
                                          segment_tokens, _ptr(saved), sv_have, _ptr(workspace),
                                          ws_have, _stream(dev))
        name = "lightning_attn_bwd_saved"
    else:
        st = lib.lightning_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(dout),
                                    _ptr(dfinal), _ptr(init_state), _ptr(dq), _ptr(dk), _ptr(dv),
                                    _ptr(dinit), B, H, N, d, block, dt, layout, segment_tokens,
                                    _ptr(workspace), ws_have, _stream(dev))
        name = "lightning_attn_bwd"
    if st != 0:
        raise LightningAttnError(st, name)
    return dq, dk, dv, dinit


def lightning_attn_fwd_chdecay_workspace_size(B, H, N, d, block=128, dtype=LA_BF16,
                                              segment_tokens=0):
    return load_library().lightning_attn_fwd_chdecay_workspace_size(B, H, N, d, block, dtype,
                                                                     segment_tokens)


def lightning_attn_fwd_chdecay(q, k, v, alpha, layout=LA_HEAD_MAJOR, block=128, init_state=None,
                               segment_tokens=0, out=None, final_state=None, workspace=None):
    """Channel-wise decay: alpha [H, d] float32 holds one decay per key
    channel of each head.  q, k, v as for lightning_attn_fwd_layout.  Returns
    (out, final_state [B, H, d, d] float32)."""
    torch = _torch()
    lib = load_library()
    if layout == LA_TOKEN_MAJOR:
        B, N, H, d = q.shape
    elif layout == LA_HEAD_MAJOR:
        B, H, N, d = q.shape
    else:
        raise ValueError("layout must be LA_HEAD_MAJOR or LA_TOKEN_MAJOR")
    dev = q.device
    for t, n in ((k, "k"), (v, "v"), (q, "q")):
        _check(t, n, q.shape, q.dtype, dev)
    _check(alpha, "alpha", (H, d), torch.float32, dev)
    if init_state is not None:
        _check(init_state, "init_state", (B, H, d, d), torch.float32, dev)
    out = torch.empty_like(q) if out is None else out
    _check(out, "out", q.shape, q.dtype, dev)
    if final_state is None:
        final_state = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    _check(final_state, "final_state", (B, H, d, d), torch.float32, dev)
    dt = _dtype_code(q)
    ws_bytes = lib.lightning_attn_fwd_chdecay_workspace_size(B, H, N, d, block, dt,
                                                             segment_tokens)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.lightning_attn_fwd_chdecay(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), B, H, N, d, block,
                                        dt, layout, _ptr(init_state), _ptr(out), _ptr(final_state),
                                        segment_tokens, _ptr(workspace), ws_have, _stream(dev))
    if st != 0:
        raise LightningAttnError(st, "lightning_attn_fwd_chdecay")
    return out, final_state


def lightning_attn_fwd_chdecay_varlen_workspace_size(num_seqs, H, total, d, block=128,
                                                     dtype=LA_BF16, segment_tokens=0):
    return load_library().lightning_attn_fwd_chdecay_varlen_workspace_size(
        num_seqs, H, total, d, block, dtype, segment_tokens)


def lightning_attn_fwd_chdecay_varlen(q, k, v, alpha, cu_seqlens, layout=LA_HEAD_MAJOR, block=128,
                                      init_states=None, segment_tokens=0, out=None,
                                      final_states=None, workspace=None):
    """Channel-wise decay over packed sequences: q, k, v [H, total, d]
    (LA_HEAD_MAJOR) or [total, H, d] (LA_TOKEN_MAJOR), alpha [H, d] float32,
    cu_seqlens int32 [num_seqs + 1].  Returns (out, final_states
    [num_seqs, H, d, d] float32)."""
    torch = _torch()
    lib = load_library()
    if layout == LA_TOKEN_MAJOR:
        total, H, d = q.shape
    elif layout == LA_HEAD_MAJOR:
        H, total, d = q.shape
    else:
        raise ValueError("layout must be LA_HEAD_MAJOR or LA_TOKEN_MAJOR")
    dev = q.device
    for t, n in ((k, "k"), (v, "v"), (q, "q")):
        _check(t, n, q.shape, q.dtype, dev)
    _check(alpha, "alpha", (H, d), torch.float32, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of num_seqs + 1 offsets")
    S = cu_seqlens.numel() - 1
    _check(cu_seqlens, "cu_seqlens", (S + 1,), torch.int32, dev)
    if init_states is not None:
        _check(init_states, "init_states", (S, H, d, d), torch.float32, dev)
    out = torch.empty_like(q) if out is None else out
    _check(out, "out", q.shape, q.dtype, dev)
    if final_states is None:
        final_states = torch.empty((S, H, d, d), dtype=torch.float32, device=dev)
    _check(final_states, "final_states", (S, H, d, d), torch.float32, dev)
    dt = _dtype_code(q)
    ws_bytes = lib.lightning_attn_fwd_chdecay_varlen_workspace_size(S, H, total, d, block, dt,
                                                                     segment_tokens)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.lightning_attn_fwd_chdecay_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                               _ptr(cu_seqlens), S, H, total, d, block, dt, layout,
                                               _ptr(init_states), _ptr(out), _ptr(final_states),
                                               segment_tokens, _ptr(workspace), ws_have,
                                               _stream(dev))
    if st != 0:
        raise LightningAttnError(st, "lightning_attn_fwd_chdecay_varlen")
    return out, final_states


def lightning_attn_bwd_varlen_workspace_size(num_seqs, H, total, d, block=128, dtype=LA_BF16,
                                             segment_tokens=0):
    return load_library().lightning_attn_bwd_varlen_workspace_size(num_seqs, H, total, d, block,
                                                                    dtype, segment_tokens)


def lightning_attn_bwd_varlen(q, k, v, decay, dout, cu_seqlens, layout=LA_HEAD_MAJOR, block=128,
                              dfinals=None, init_states=None, segment_tokens=0, want_dinit=True,
                              dq=None, dk=None, dv=None, dinits=None, workspace=None):
    """Gradients of lightning_attn_fwd_varlen_layout: q, k, v, dout
    [H, total, d] (LA_HEAD_MAJOR) or [total, H, d] (LA_TOKEN_MAJOR);
    cu_seqlens int32 [num_seqs + 1]; dfinals and init_states
    [num_seqs, H, d, d] float32 or None.  Returns (dq, dk, dv, dinits)."""
    return _bwd_varlen(q, k, v, decay, dout, cu_seqlens, layout, block, dfinals, init_states,
                       segment_tokens, want_dinit, dq, dk, dv, dinits, workspace, False, None)


def lightning_attn_bwd_varlen_saved(q, k, v, decay, dout, cu_seqlens, saved, layout=LA_HEAD_MAJOR,
                                    block=128, dfinals=None, init_states=None, segment_tokens=0,
                                    want_dinit=True, dq=None, dk=None, dv=None, dinits=None,
                                    workspace=None):
    """lightning_attn_bwd_varlen with the segment states `saved` kept by
    lightning_attn_fwd_varlen_save on the same inputs and arguments."""
    return _bwd_varlen(q, k, v, decay, dout, cu_seqlens, layout, block, dfinals, init_states,
                       segment_tokens, want_dinit, dq, dk, dv, dinits, workspace, True, saved)


def lightning_attn_varlen_saved_states_size(num_seqs, H, total, d, block=128, dtype=LA_BF16,
                                            segment_tokens=0):
    return load_library().lightning_attn_varlen_saved_states_size(num_seqs, H, total, d, block,
                                                                   dtype, segment_tokens)


def lightning_attn_fwd_varlen_save(q, k, v, decay, cu_seqlens, layout=LA_HEAD_MAJOR, block=128,
                                   init_states=None, segment_tokens=0, out=None,
                                   final_states=None, saved=None, workspace=None):
    """The packed forward of a training pair (see lightning_attn_fwd_save).
    Returns (out, final_states, saved); the workspace is sized by
    lightning_attn_bwd_varlen_workspace_size."""
    torch = _torch()
    lib = load_library()
    if layout == LA_TOKEN_MAJOR:
        total, H, d = q.shape
    elif layout == LA_HEAD_MAJOR:
        H, total, d = q.shape
    else:
        raise ValueError("layout must be LA_HEAD_MAJOR or LA_TOKEN_MAJOR")
    dev = q.device
    for t, n in ((k, "k"), (v, "v"), (q, "q")):
        _check(t, n, q.shape, q.dtype, dev)
    _check(decay, "decay", (H,), torch.float32, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of num_seqs + 1 offsets")
    S = cu_seqlens.numel() - 1
    _check(cu_seqlens, "cu_seqlens", (S + 1,), torch.int32, dev)
    if init_states is not None:
        _check(init_states, "init_states", (S, H, d, d), torch.float32, dev)
    out = torch.empty_like(q) if out is None else out
    _check(out, "out", q.shape, q.dtype, dev)
    if final_states is None:
        final_states = torch.empty((S, H, d, d), dtype=torch.float32, device=dev)
    _check(final_states, "final_states", (S, H, d, d), torch.float32, dev)
    dt = _dtype_code(q)
    sv_bytes = lib.lightning_attn_varlen_saved_states_size(S, H, total, d, block, dt,
                                                           segment_tokens)
    if saved is None and sv_bytes:
        saved = torch.empty(sv_bytes // 4, dtype=torch.float32, device=dev)
    sv_have = saved.numel() * saved.element_size() if saved is not None else 0
    ws_bytes = lib.lightning_attn_bwd_varlen_workspace_size(S, H, total, d, block, dt,
                                                             segment_tokens)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.lightning_attn_fwd_varlen_save(_ptr(q), _ptr(k), _ptr(v), _ptr(decay),
                                            _ptr(cu_seqlens), S, H, total, d, block, dt, layout,
                                            _ptr(init_states), _ptr(out), _ptr(final_states),
                                            segment_tokens, _ptr(saved), sv_have,
                                            _ptr(workspace), ws_have, _stream(dev))
    if st != 0:
        raise LightningAttnError(st, "lightning_attn_fwd_varlen_save")
    return out, final_states, saved


def _bwd_varlen(q, k, v, decay, dout, cu_seqlens, layout, block, dfinals, init_states,
                segment_tokens, want_dinit, dq, dk, dv, dinits, workspace, with_saved, saved):
    torch = _torch()
    lib = load_library()
    if layout == LA_TOKEN_MAJOR:
        total, H, d = q.shape
    elif layout == LA_HEAD_MAJOR:
        H, total, d = q.shape
    else:
        raise ValueError("layout must be LA_HEAD_MAJOR or LA_TOKEN_MAJOR")
    dev = q.device
    for t, n in ((k, "k"), (v, "v"), (dout, "dout"), (q, "q")):
        _check(t, n, q.shape, q.dtype, dev)
    _check(decay, "decay", (H,), torch.float32, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of num_seqs + 1 offsets")
    S = cu_seqlens.numel() - 1
    _check(cu_seqlens, "cu_seqlens", (S + 1,), torch.int32, dev)
    for t, n in ((dfinals, "dfinals"), (init_states, "init_states")):
        if t is not None:
            _check(t, n, (S, H, d, d), torch.float32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, n, q.shape, q.dtype, dev)
    if want_dinit and dinits is None:
        dinits = torch.empty((S, H, d, d), dtype=torch.float32, device=dev)
    if dinits is not None:
        _check(dinits, "dinits", (S, H, d, d), torch.float32, dev)
    dt = _dtype_code(q)
    ws_bytes = lib.lightning_attn_bwd_varlen_workspace_size(S, H, total, d, block, dt,
                                                             segment_tokens)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if with_saved:
        if saved is not None:
            _check(saved, "saved", saved.shape, torch.float32, dev)
        sv_have = saved.numel() * saved.element_size() if saved is not None else 0
        st = lib.lightning_attn_bwd_varlen_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(decay),
                                                 _ptr(dout), _ptr(cu_seqlens), S, H, total, d,
                                                 block, dt, layout, _ptr(dfinals),
                                                 _ptr(init_states), _ptr(dq), _ptr(dk), _ptr(dv),
                                                 _ptr(dinits), segment_tokens, _ptr(saved),
                                                 sv_have, _ptr(workspace), ws_have, _stream(dev))
        name = "lightning_attn_bwd_varlen_saved"
    else:
        st = lib.lightning_attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(dout),
                                           _ptr(cu_seqlens), S, H, total, d, block, dt, layout,
                                           _ptr(dfinals), _ptr(init_states), _ptr(dq), _ptr(dk),
                                           _ptr(dv), _ptr(dinits), segment_tokens,
                                           _ptr(workspace), ws_have, _stream(dev))
        name = "lightning_attn_bwd_varlen"
    if st != 0:
        raise LightningAttnError(st, name)
    return dq, dk, dv, dinits
