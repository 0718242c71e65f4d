"""Seeded synthetic inputs for lightning attention.

This module draws random numbers and builds the per-head decay schedule; it
holds none of the attention arithmetic, so the HIP path's tests, the CPU
oracle's tests and the benchmark can all take their inputs from it.

Recipe (all synthetic; no dataset is involved):
  * q, k, v ~ N(0, 1) / sqrt(d), drawn in float32, then rounded to bf16
    (round-to-nearest-even) for bf16 workloads.  The oracle receives the
    rounded values, widened back to float32 (exact).
  * decay lambda_h = exp(-2^(-8 (h + 1) / H)) for head h = 0 .. H-1, computed
    in float64 and rounded once to float32; both sides use that float32.
  * decode state ~ N(0, 0.1^2) in float32 (variance 0.01).
  * packed variable-length batches: lognormal lengths with median 2048
    (mu = ln 2048, sigma = 1), rounded to the nearest integer, clipped to
    [1, 32768], drawn until the total reaches the target and the last one
    truncated so the total is exact.

Two generators: ``host_*`` uses numpy's PCG64 (CPU tests, small cases) and
``device_*`` uses torch's Philox generator on the GPU (large cases, where
drawing on the host would dominate).  Both are seeded; a given (seed, shape,
backend) always yields the same values.
"""
import math

import numpy as np

# The five workloads: (name, kind, sizes).
WORKLOADS = {
    "tiny_fp32": dict(kind="fwd", B=1, H=2, N=256, d=64, block=64, dtype="fp32", seed=1),
    "mid_bf16": dict(kind="fwd", B=2, H=8, N=4096, d=128, block=64, dtype="bf16", seed=2),
    "layer_h64_n32k": dict(kind="fwd", B=1, H=64, N=32768, d=128, block=128, dtype="bf16",
                           seed=3),
    "layer_h64_varlen64k": dict(kind="varlen", H=64, total=65536, d=128, block=128,
                                dtype="bf16", seed=33),
    "million_h8": dict(kind="fwd", B=1, H=8, N=1048576, d=128, block=256, dtype="bf16",
                       seed=4),
    "decode_b128_h64": dict(kind="decode", B=128, H=64, d=128, steps=256, dtype="bf16",
                            seed=5),
}


def decay_schedule(H):
    """float32 lambda_h = exp(-2^(-8 (h+1) / H)), h = 0 .. H-1."""
    lam = [math.exp(-(2.0 ** (-8.0 * (h + 1) / H))) for h in range(H)]
    return np.asarray(lam, dtype=np.float64).astype(np.float32)


def chdecay_schedule(H, d, seed=7):
    """float32 per-channel decays [H, d] for the channel-wise variant: around
    head h's scalar rate 2^(-8 (h+1) / H), channel i decays at that rate times
    2^u_i with u_i ~ U(-3, 1) (seeded), alpha = exp(-rate) -- a head's
    channels span 16x in decay rate, all alpha >= 0.15; channel 0 of every
    head is exactly 1."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(-3.0, 1.0, (H, d))
    rate = (2.0 ** (-8.0 * (np.arange(H)[:, None] + 1) / H)) * 2.0 ** u
    a = np.exp(-rate)
    a[:, 0] = 1.0
    return a.astype(np.float32)


def round_to_bf16(x):
    """Round float32 values to the nearest bf16 (ties to even); returns the
    rounded values as float32 (every bf16 is exactly a float32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(x)
    out = r.astype(np.uint32).view(np.float32)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out.reshape(x.shape)


def host_qkv(shape, seed, dtype="bf16"):
    """(q, k, v) float32 numpy arrays of `shape` (last dim d), each
    N(0, 1)/sqrt(d), rounded to bf16 values when dtype == "bf16"."""
    d = shape[-1]
    ss = np.random.SeedSequence(seed)
    outs = []
    for child in ss.spawn(3):
        g = np.random.Generator(np.random.PCG64(child))
        x = (g.standard_normal(shape, dtype=np.float32) / np.float32(math.sqrt(d)))
        outs.append(round_to_bf16(x) if dtype == "bf16" else x.astype(np.float32))
    return tuple(outs)


def host_state(shape, seed, std=0.1):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def varlen_lengths(total=65536, median=2048, sigma=1.0, max_len=32768, seed=33):
    """Lognormal sequence lengths summing exactly to `total`."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    mu = math.log(median)
    lens, s = [], 0
    while s < total:
        n = int(round(math.exp(mu + sigma * float(g.standard_normal()))))
        n = max(1, min(max_len, n))
        n = min(n, total - s)
        lens.append(n)
        s += n
    return lens


def cu_seqlens(lengths):
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def device_qkv(shape, seed, dtype="bf16", device="cuda"):
    """(q, k, v) torch tensors on `device`, N(0, 1)/sqrt(d) drawn in float32
    with torch's seeded Philox generator, then cast (round-to-nearest-even)
    to bf16 when dtype == "bf16"."""
    import torch
    d = shape[-1]
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    outs = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        x.mul_(1.0 / math.sqrt(d))
        outs.append(x.to(tdt))
    return tuple(outs)


def device_state(shape, seed, std=0.1, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.mul_(std)
