"""The allocation-free prefill (lightning_attn_fwd_noalloc), called through
the C ABI, against lightning_attn_fwd with a caller workspace: the two run
the same kernels on the same inputs, so their outputs and final states must
be bit-identical -- on two calls in a row, the second with a smaller input,
for the three-phase and the single-pass schedules and the vector-ALU path;
and a call that needs more scratch than the library holds is refused before
anything launches."""
import ctypes

import numpy as np
import pytest

import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import inputs

pytestmark = pytest.mark.gpu


def torch_mod():
    import torch
    return torch


def noalloc_c(q, k, v, decay, out, fin, init=None, seg=0, block=128):
    """lightning_attn_fwd_noalloc straight through ctypes."""
    torch = torch_mod()
    lib = la.load_library()
    B, H, N, d = q.shape
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    dt = 1 if q.dtype == torch.bfloat16 else 0
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.lightning_attn_fwd_noalloc(P(q), P(k), P(v), P(decay), B, H, N, d, block, dt,
                                          P(init), P(out), P(fin), seg, stream)


def one_case(B, H, N, d, dtype, seed, seg, with_init):
    torch = torch_mod()
    print("case noalloc B=%d H=%d N=%d d=%d %s seg=%d init=%s" % (B, H, N, d, dtype, seg,
                                                                    with_init), flush=True)
    tq, tk, tv = inputs.device_qkv((B, H, N, d), seed, dtype)
    tl = torch.from_numpy(inputs.decay_schedule(H)).cuda()
    ti = inputs.device_state((B, H, d, d), seed + 1) if with_init else None
    need = la.lightning_attn_fwd_workspace_size(B, H, N, d, 128, la._dtype_code(tq), seg)
    assert need <= la.lightning_attn_noalloc_scratch_bytes()
    ref_out, ref_fin = la.lightning_attn_fwd(tq, tk, tv, tl, init_state=ti, segment_tokens=seg)
    out = torch.full_like(tq, float("nan"))
    fin = torch.full((B, H, d, d), float("nan"), device="cuda")
    assert noalloc_c(tq, tk, tv, tl, out, fin, init=ti, seg=seg) == 0
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(fin, ref_fin)
    # and through the Python binding
    out2, fin2 = la.lightning_attn_fwd_noalloc(tq, tk, tv, tl, init_state=ti, segment_tokens=seg)
    torch.cuda.synchronize()
    assert torch.equal(out2, ref_out) and torch.equal(fin2, ref_fin)
    return need


@pytest.mark.parametrize("path", ["phased", "fused"])
def test_noalloc_matches_fwd_on_two_calls(path, monkeypatch):
    """The headline shape (whose plan fills the whole scratch array), then a
    smaller call with segment cuts and an initial state: the second call
    finds the first one's partial states and flags left in the array."""
    monkeypatch.setenv("LIGHTNING_ATTN_PREFILL", path)
    n1 = one_case(1, 64, 32768, 128, "bf16", seed=3, seg=0, with_init=False)
    n2 = one_case(2, 8, 3000, 128, "bf16", seed=11, seg=512, with_init=True)
    assert n2 < n1


def test_noalloc_vector_alu_path():
    one_case(1, 3, 1000, 64, "fp32", seed=13, seg=256, with_init=True)
    one_case(1, 2, 300, 64, "fp32", seed=14, seg=128, with_init=False)


def test_noalloc_refuses_beyond_scratch():
    """32-token segments over 64 heads need 512 MiB of partial states: the
    call returns LA_ERR_WORKSPACE and writes nothing."""
    torch = torch_mod()
    B, H, N, d = 1, 64, 4096, 128
    need = la.lightning_attn_fwd_workspace_size(B, H, N, d, 128, 1, 32)
    assert need > la.lightning_attn_noalloc_scratch_bytes()
    tq, tk, tv = inputs.device_qkv((B, H, N, d), 15, "bf16")
    tl = torch.from_numpy(inputs.decay_schedule(H)).cuda()
    out = torch.full_like(tq, float("nan"))
    fin = torch.full((B, H, d, d), float("nan"), device="cuda")
    assert noalloc_c(tq, tk, tv, tl, out, fin, seg=32) == 3
    torch.cuda.synchronize()
    assert bool(torch.isnan(out).all()) and bool(torch.isnan(fin).all())
    with pytest.raises(la.LightningAttnError, match="LA_ERR_WORKSPACE"):
        la.lightning_attn_fwd_noalloc(tq, tk, tv, tl, segment_tokens=32)
