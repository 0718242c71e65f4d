"""Benchmark: lightning attention prefill (and decode) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]

A step is one prefill pass of the headline workload -- B=1, H=64, N=32768,
d=128, block 128, bf16 inputs, float32 state -- through the C ABI, with its
inputs already resident in HBM.  W untimed steps, then K steps timed with
HIP events on the stream the library launches on.  Prints ONE JSON line:
the headline tokens/s, TFLOP/s and fraction of the bf16 MFMA peak, the HBM
roofline of the step, the CPU oracle timed on a bounded sample, and (unless
--no-extras) the decode, packed varlen, million-token, token-major, backward,
channel-wise, prefix-snapshot, short-chunk/gated and mixed serving-step
workloads, and last the headline step re-timed after all of them
(steady_state: the settled clock, with the per-step median and minimum).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s & TFLOP/s (% MFMA peak) at H=64 d=128; decode state GB/s"
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def prefill_flops(B, H, N, d, C):
    """Dense-block FLOPs of the blockwise form: Q K^T and P V inside blocks
    (4 C d per token) plus Q S and K^T V per token (4 d^2)."""
    return B * H * N * 4 * d * (C + d)


def prefill_bytes(B, H, N, d, in_bytes=2, out_bytes=2):
    """Algorithmic HBM bytes: q, k, v read once, out written once, final
    state written once, decay read once."""
    return B * H * N * d * (3 * in_bytes + out_bytes) + B * H * d * d * 4 + 4 * H


def decode_bytes(B, H, d, io_bytes=2):
    """Per decode step: the float32 state read and written once, plus q, k,
    v and out."""
    return 2 * B * H * d * d * 4 + 4 * B * H * d * io_bytes


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_lightning_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes from the committed rocprofv3 counter summary (scaled FETCH_SIZE
    + WRITE_SIZE), if it was taken on the current kernel sources; else None.
    Returns {"step": bytes per step, kernel name: bytes per launch, ...}."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    out = dict(rec.get("kernels", {}))
    out["step"] = rec.get("bytes_per_step")
    return out


def time_steps(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per step


def bench_prefill(la, inputs, B, H, N, d, block, seed, steps, warmup, phases=False, trace=None):
    """ms per step over `steps` timed steps after `warmup`.  With phases, also
    the average ms of each of the library's three phases (local-state pass,
    segment scan, output pass), from HIP events the library records between
    its launches on the same stream, on every fifth timed step (the last one
    if there are fewer than five).  Recording events between launches leaves
    short gaps in which the clock recovers; sampling a few steps keeps the
    sampled kernels in the same sustained state as the rest and the step time
    nearly undisturbed (the step time includes those few gaps)."""
    import torch
    dev = torch.device("cuda:0")
    q, k, v = inputs.device_qkv((B, H, N, d), seed, "bf16", device=dev)
    decay = torch.from_numpy(inputs.decay_schedule(H)).to(dev)
    out = torch.empty_like(q)
    fin = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    nws = la.lightning_attn_fwd_workspace_size(B, H, N, d, block)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sampled = [i for i in range(steps) if (i + 1) % 5 == 0] or [steps - 1]
    evs = {}
    if phases:
        for i in sampled:
            evs[i] = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            for e in evs[i]:
                e.record(stream)  # creates the event, so that its handle exists
    calls = [0]

    def step():
        i = calls[0] - warmup
        calls[0] += 1
        if i in evs:
            la.lightning_attn_fwd_timed(q, k, v, decay, [e.cuda_event for e in evs[i]],
                                        block=block, out=out, final_state=fin, workspace=ws)
        else:
            la.lightning_attn_fwd(q, k, v, decay, block=block, out=out, final_state=fin,
                                  workspace=ws)

    run = step
    if trace is not None:
        # An event after every step, the warm-up included (diagnostic: the
        # records between launches leave short gaps of their own).
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(warmup + steps + 1)]

        def run():
            step()
            marks[calls[0]].record(stream)

        torch.cuda.synchronize()
        marks[0].record(stream)
    ms = time_steps(run, steps, warmup, stream)
    if trace is not None:
        trace.extend(round(marks[i].elapsed_time(marks[i + 1]) * 1e3, 1)
                     for i in range(warmup + steps))
    phase_ms = None
    if phases:
        phase_ms = [sum(row[j].elapsed_time(row[j + 1]) for row in evs.values()) / len(evs)
                    for j in range(3)]
    return ms, phase_ms, (q, k, v, decay, out, fin)


STEADY_WARMUP = 60


def bench_steady(la, inputs, w, steps):
    """The headline step again at the end of the run, after STEADY_WARMUP
    warm-up steps: past the clock transient that follows the start of
    sustained work (it recurs after the light serving legs, so the warm-up is
    its own, not --warmup).  The same number of timed steps as the headline,
    with the phases sampled the same way; then as many steps again, each
    between two HIP events, for the per-step median and minimum (the event
    records between steps leave short gaps of their own, so those come from a
    loop of their own)."""
    warmup = STEADY_WARMUP
    B, H, N, d, block = w["B"], w["H"], w["N"], w["d"], w["block"]
    ms, phase_ms, tensors = bench_prefill(la, inputs, B, H, N, d, block, w["seed"], steps,
                                          warmup, phases=True)
    del tensors
    trace = []
    bench_prefill(la, inputs, B, H, N, d, block, w["seed"], steps, 0, trace=trace)
    per_step = sorted(trace)
    alg = prefill_bytes(B, H, N, d)
    median = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    return {"workload": "layer_h64_n32k", "when": "after every other leg",
            "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(B * N / (ms * 1e-3), 1),
            "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "chunk_kernel_us": round(phase_ms[2] * 1e3, 1),
            "chunk_kernel_frac": round(alg / (phase_ms[2] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "local_state_us": round(phase_ms[0] * 1e3, 1),
            "scan_us": round(phase_ms[1] * 1e3, 1),
            "per_step_ms_median": round(median * 1e-3, 4),
            "per_step_ms_min": round(per_step[0] * 1e-3, 4),
            "note": "the headline step re-timed at the end of the run after its own "
                    "warm-up; value and roofline above are the first measurement, straight "
                    "after start-up with --warmup steps"}


def bench_token_major(la, inputs, steps, warmup):
    """The headline workload with q, k, v, out in [B, N, H, d] layout (a
    projection's output, read in place through a row stride)."""
    import torch
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS["layer_h64_n32k"]
    B, H, N, d, block = w["B"], w["H"], w["N"], w["d"], w["block"]
    q, k, v = (t.transpose(1, 2).contiguous()
               for t in inputs.device_qkv((B, H, N, d), w["seed"], "bf16", device=dev))
    decay = torch.from_numpy(inputs.decay_schedule(H)).to(dev)
    out = torch.empty_like(q)
    fin = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    nws = la.lightning_attn_fwd_workspace_size(B, H, N, d, block)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def step():
        la.lightning_attn_fwd_layout(q, k, v, decay, la.LA_TOKEN_MAJOR, block=block, out=out,
                                     final_state=fin, workspace=ws)

    ms = time_steps(step, steps, warmup, torch.cuda.current_stream(dev))
    byt = prefill_bytes(B, H, N, d)
    return {"workload": "layer_h64_n32k", "layout": "token-major [B, N, H, d]",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(B * N / (ms * 1e-3), 1),
            "hbm_gbs_algorithmic": round(byt / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def bench_varlen(la, inputs, steps, warmup):
    import torch
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS["layer_h64_varlen64k"]
    H, total, d, block = w["H"], w["total"], w["d"], w["block"]
    lens = inputs.varlen_lengths(total=total, seed=w["seed"])
    cu = torch.from_numpy(inputs.cu_seqlens(lens)).to(dev)
    q, k, v = inputs.device_qkv((H, total, d), w["seed"], "bf16", device=dev)
    decay = torch.from_numpy(inputs.decay_schedule(H)).to(dev)
    out = torch.empty_like(q)
    fin = torch.empty((len(lens), H, d, d), dtype=torch.float32, device=dev)
    nws = la.lightning_attn_fwd_varlen_workspace_size(len(lens), H, total, d, block)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def step():
        la.lightning_attn_fwd_varlen(q, k, v, decay, cu, block=block, out=out, final_states=fin,
                                     workspace=ws)

    ms = time_steps(step, steps, warmup, torch.cuda.current_stream(dev))
    byt = H * total * d * 8 + len(lens) * H * d * d * 4
    return {"workload": "layer_h64_varlen64k", "num_seqs": len(lens), "H": H, "total": total,
            "ms_per_step": round(ms, 4), "tokens_per_s": round(total / (ms * 1e-3), 1),
            "tflops": round(prefill_flops(1, H, total, d, 128) / (ms * 1e-3) / 1e12, 2),
            "hbm_gbs_algorithmic": round(byt / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def bench_million(la, inputs, steps, warmup):
    w = inputs.WORKLOADS["million_h8"]
    B, H, N, d, block = w["B"], w["H"], w["N"], w["d"], w["block"]
    ms, _, _ = bench_prefill(la, inputs, B, H, N, d, block, w["seed"], steps, warmup)
    byt = prefill_bytes(B, H, N, d)
    return {"workload": "million_h8", "B": B, "H": H, "N": N, "block": block,
            "ms_per_step": round(ms, 4), "tokens_per_s": round(B * N / (ms * 1e-3), 1),
            "tflops_at_block": round(prefill_flops(B, H, N, d, block) / (ms * 1e-3) / 1e12, 2),
            "tflops_executed_chunk128": round(prefill_flops(B, H, N, d, 128) / (ms * 1e-3) / 1e12, 2),
            "hbm_gbs_algorithmic": round(byt / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def bench_decode(la, inputs, reps, warmup):
    import torch
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS["decode_b128_h64"]
    B, H, d, T = w["B"], w["H"], w["d"], w["steps"]
    q, k, v = inputs.device_qkv((T, B, H, d), w["seed"], "bf16", device=dev)
    decay = torch.from_numpy(inputs.decay_schedule(H)).to(dev)
    state0 = inputs.device_state((B, H, d, d), w["seed"] + 1, device=dev)
    state = state0.clone()
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run():  # 256 consecutive one-token steps
        for t in range(T):
            la.lightning_attn_decode(q[t], k[t], v[t], decay, state, out=out)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        state.copy_(state0)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        run()
        e.record(stream)
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    times.sort()
    ms = times[len(times) // 2] / T      # median repetition
    ms_min = times[0] / T
    gbs = decode_bytes(B, H, d) / (ms * 1e-3) / 1e9
    gbs_max = decode_bytes(B, H, d) / (ms_min * 1e-3) / 1e9
    return {"workload": "decode_b128_h64", "B": B, "H": H, "d": d, "steps": T,
            "repetitions": reps, "ms_per_token_step": round(ms, 5),
            "ms_per_token_step_min": round(ms_min, 5), "state_gbs": round(gbs, 1),
            "state_gbs_best": round(gbs_max, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "note": "median (and best) of the repetitions, each 256 steps"}


def bench_backward(la, inputs, steps, warmup):
    """Backward pass (lightning_attn_bwd) at the headline shape, B=1 H=64
    N=32768 d=128 bf16, with a final-state gradient and an initial state:
    ms per step; algorithmic bytes = q, k, v, dout read and dq, dk, dv written
    once (7 x B H N d x 2 bytes, plus the d x d states)."""
    import torch
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS["layer_h64_n32k"]
    B, H, N, d, block = w["B"], w["H"], w["N"], w["d"], w["block"]
    q, k, v = inputs.device_qkv((B, H, N, d), w["seed"], "bf16", device=dev)
    do, _, _ = inputs.device_qkv((B, H, N, d), w["seed"] + 7, "bf16", device=dev)
    decay = torch.from_numpy(inputs.decay_schedule(H)).to(dev)
    init = inputs.device_state((B, H, d, d), w["seed"] + 8, device=dev)
    dfin = inputs.device_state((B, H, d, d), w["seed"] + 9, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dinit = torch.empty_like(init)
    nws = la.lightning_attn_bwd_workspace_size(B, H, N, d, block)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def step():
        la.lightning_attn_bwd(q, k, v, decay, do, dfinal=dfin, init_state=init, block=block,
                              dq=dq, dk=dk, dv=dv, dinit=dinit, workspace=ws)

    ms = time_steps(step, steps, warmup, torch.cuda.current_stream(dev))
    # The training pair: the forward keeps its segment entering states, and
    # the backward's dq pass skips its local-state pass and scan.
    _, _, saved = la.lightning_attn_fwd_save(q, k, v, decay, block=block, init_state=init,
                                             workspace=ws)

    def step_saved():
        la.lightning_attn_bwd_saved(q, k, v, decay, do, saved, dfinal=dfin, init_state=init,
                                    block=block, dq=dq, dk=dk, dv=dv, dinit=dinit, workspace=ws)

    ms_saved = time_steps(step_saved, steps, warmup, torch.cuda.current_stream(dev))
    byt = 7 * B * H * N * d * 2 + 3 * B * H * d * d * 4
    return {"workload": "layer_h64_n32k", "pass": "backward (dq, dk, dv, dinit)",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(B * N / (ms * 1e-3), 1),
            "tflops_3_passes": round(3 * prefill_flops(B, H, N, d, 128) / (ms * 1e-3) / 1e12, 2),
            "hbm_gbs_algorithmic": round(byt / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "with_saved_states": {"ms_per_step": round(ms_saved, 4),
                                  "tokens_per_s": round(B * N / (ms_saved * 1e-3), 1),
                                  "hbm_frac": round(byt / (ms_saved * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                                    4)}}


def bench_backward_varlen(la, inputs, steps, warmup):
    """Packed backward (lightning_attn_bwd_varlen) over the 65536-token
    packed workload at 64 heads (lognormal lengths, as the packed prefill),
    with final-state gradients and initial states, plain and with the
    forward's saved states: ms per step; algorithmic bytes as the
    fixed-length backward's."""
    import torch
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS["layer_h64_varlen64k"]
    H, total, d, block = w["H"], w["total"], w["d"], w["block"]
    lens = inputs.varlen_lengths(total=total, seed=w["seed"])
    S = len(lens)
    cu = torch.from_numpy(inputs.cu_seqlens(lens)).to(dev)
    q, k, v = inputs.device_qkv((H, total, d), w["seed"], "bf16", device=dev)
    do, _, _ = inputs.device_qkv((H, total, d), w["seed"] + 7, "bf16", device=dev)
    decay = torch.from_numpy(inputs.decay_schedule(H)).to(dev)
    init = inputs.device_state((S, H, d, d), w["seed"] + 8, device=dev)
    dfin = inputs.device_state((S, H, d, d), w["seed"] + 9, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dinit = torch.empty_like(init)
    nws = la.lightning_attn_bwd_varlen_workspace_size(S, H, total, d, block)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def step():
        la.lightning_attn_bwd_varlen(q, k, v, decay, do, cu, block=block, dfinals=dfin,
                                     init_states=init, dq=dq, dk=dk, dv=dv, dinits=dinit,
                                     workspace=ws)

    ms = time_steps(step, steps, warmup, torch.cuda.current_stream(dev))
    _, _, saved = la.lightning_attn_fwd_varlen_save(q, k, v, decay, cu, block=block,
                                                    init_states=init, workspace=ws)

    def step_saved():
        la.lightning_attn_bwd_varlen_saved(q, k, v, decay, do, cu, saved, block=block,
                                           dfinals=dfin, init_states=init, dq=dq, dk=dk, dv=dv,
                                           dinits=dinit, workspace=ws)

    ms_saved = time_steps(step_saved, steps, warmup, torch.cuda.current_stream(dev))
    byt = 7 * H * total * d * 2 + 3 * S * H * d * d * 4
    return {"workload": "layer_h64_varlen64k", "pass": "packed backward (dq, dk, dv, dinit)",
            "num_seqs": S, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(total / (ms * 1e-3), 1),
            "hbm_gbs_algorithmic": round(byt / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "with_saved_states": {"ms_per_step": round(ms_saved, 4),
                                  "tokens_per_s": round(total / (ms_saved * 1e-3), 1),
                                  "hbm_frac": round(byt / (ms_saved * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                                    4)}}


def bench_chdecay(la, inputs, steps, warmup):
    """Channel-wise decay prefill at the headline shape (B=1 H=64 N=32768
    d=128 bf16, per-channel decays from inputs.chdecay_schedule): ms per step,
    tokens/s, algorithmic HBM bytes (as the scalar prefill) and the bf16 MFMA
    rate at the formula 4 d (C + d) per token-head with the kernel's
    64-token chunk."""
    import torch
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS["layer_h64_n32k"]
    B, H, N, d, block = w["B"], w["H"], w["N"], w["d"], w["block"]
    q, k, v = inputs.device_qkv((B, H, N, d), w["seed"], "bf16", device=dev)
    alpha = torch.from_numpy(inputs.chdecay_schedule(H, d)).to(dev)
    out = torch.empty_like(q)
    fin = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    nws = la.lightning_attn_fwd_chdecay_workspace_size(B, H, N, d, block)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def step():
        la.lightning_attn_fwd_chdecay(q, k, v, alpha, block=block, out=out, final_state=fin,
                                      workspace=ws)

    ms = time_steps(step, steps, warmup, torch.cuda.current_stream(dev))
    byt = prefill_bytes(B, H, N, d)
    return {"workload": "layer_h64_n32k", "decay": "channel-wise [H, d]",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(B * N / (ms * 1e-3), 1),
            "tflops_chunk64": round(prefill_flops(B, H, N, d, 64) / (ms * 1e-3) / 1e12, 2),
            "mfma_peak_frac": round(prefill_flops(B, H, N, d, 64) / (ms * 1e-3) / 1e12
                                    / PEAK_BF16_TFLOPS, 4),
            "hbm_gbs_algorithmic": round(byt / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def bench_snapshots(la, inputs, steps, warmup, interval=256):
    """The packed 65536-token workload with a prefix-state snapshot every
    `interval` tokens of each sequence (a prefix cache): time per step, and
    the snapshot bytes it adds to the algorithmic traffic."""
    import torch
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS["layer_h64_varlen64k"]
    H, total, d, block = w["H"], w["total"], w["d"], w["block"]
    lens = inputs.varlen_lengths(total=total, seed=w["seed"])
    cu = torch.from_numpy(inputs.cu_seqlens(lens)).to(dev)
    q, k, v = inputs.device_qkv((H, total, d), w["seed"], "bf16", device=dev)
    decay = torch.from_numpy(inputs.decay_schedule(H)).to(dev)
    out = torch.empty_like(q)
    fin = torch.empty((len(lens), H, d, d), dtype=torch.float32, device=dev)
    nws = la.lightning_attn_fwd_varlen_workspace_size(len(lens), H, total, d, block)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    offs = la.snapshot_row_offsets(cu, interval)
    toffs = torch.tensor(offs, dtype=torch.int32, device=dev)
    snaps = torch.empty((offs[-1], H, d, d), dtype=torch.float32, device=dev)

    def step():
        la.lightning_attn_fwd_varlen_snapshots(q, k, v, decay, cu, interval, block=block,
                                               out=out, final_states=fin, snapshots=snaps,
                                               snapshot_offsets=toffs, workspace=ws)

    ms = time_steps(step, steps, warmup, torch.cuda.current_stream(dev))
    snap_bytes = offs[-1] * H * d * d * 4
    byt = H * total * d * 8 + len(lens) * H * d * d * 4 + snap_bytes
    return {"workload": "layer_h64_varlen64k", "snapshot_interval": interval,
            "snapshot_rows": offs[-1], "snapshot_bytes": snap_bytes,
            "ms_per_step": round(ms, 4), "tokens_per_s": round(total / (ms * 1e-3), 1),
            "hbm_gbs_algorithmic": round(byt / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def bench_short_gated(la, inputs, steps, warmup):
    """The B=1 H=64 N=32768 layer on the short-chunk kernel (block 64 and 32)
    and through the gated path (SiLU on q, k, v, normalisation with a weight,
    sigmoid gate: every part; and none), ms per step beside block 128.
    Algorithmic bytes as the headline (the gated path also reads the gate:
    +2 bytes per element)."""
    import torch
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS["layer_h64_n32k"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    q, k, v = inputs.device_qkv((B, H, N, d), w["seed"], "bf16", device=dev)
    g, _, _ = inputs.device_qkv((B, H, N, d), w["seed"] + 9, "bf16", device=dev)
    decay = torch.from_numpy(inputs.decay_schedule(H)).to(dev)
    wgt = torch.ones((H, d), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    fin = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    res = {"workload": "layer_h64_n32k", "unit": "ms per step"}
    for block in (128, 64, 32):
        nws = la.lightning_attn_fwd_workspace_size(B, H, N, d, block)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

        def step():
            la.lightning_attn_fwd(q, k, v, decay, block=block, out=out, final_state=fin,
                                  workspace=ws)

        ms = time_steps(step, steps, warmup, stream)
        res["block_%d" % block] = {"ms_per_step": round(ms, 4),
                                   "hbm_frac": round(prefill_bytes(B, H, N, d) / (ms * 1e-3) / 1e9
                                                     / PEAK_HBM_GBS, 4)}
    allf = la.LA_SILU_Q | la.LA_SILU_K | la.LA_SILU_V | la.LA_NORM | la.LA_GATE
    nws = la.lightning_attn_fwd_gated_workspace_size(B, H, N, d)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    for name, flags in (("gated_all", allf), ("gated_none", 0)):
        def step():
            la.lightning_attn_fwd_gated(q, k, v, decay, flags, gate=g, norm_weight=wgt, out=out,
                                        final_state=fin, workspace=ws)

        ms = time_steps(step, steps, warmup, stream)
        byt = prefill_bytes(B, H, N, d) + (B * H * N * d * 2 if flags else 0)
        res[name] = {"ms_per_step": round(ms, 4),
                     "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    return res


def bench_serving(la, inputs, reps=200, P=50):
    """A mixed serving step at the 64-head layer shape: 20 sequences with
    prefix states, two continuing with P new tokens and eighteen decoding one.
    Variants: the P-token prefill alone, the decode alone, both on one stream,
    both on two streams (lightning_attn_mixed_step), and all twenty sequences
    as one packed prefill.  Prefills take one segment per sequence.  Two
    timings in microseconds per step: `eager` (median of single steps, each
    launched from Python and synchronised, so host launch gaps count) and
    `graph` (the step captured once as a HIP graph and replayed `reps` times
    back to back)."""
    import torch
    dev = torch.device("cuda:0")
    H, d, B = 64, 128, 18
    seg = la.LA_SEGMENT_PER_SEQUENCE
    plens = [P, P]
    decay = torch.from_numpy(inputs.decay_schedule(H)).to(dev)
    cu = torch.from_numpy(inputs.cu_seqlens(plens)).to(dev)
    pq, pk, pv = inputs.device_qkv((H, sum(plens), d), 401, "bf16", device=dev)
    dq, dk, dv = inputs.device_qkv((B, H, d), 402, "bf16", device=dev)
    pinit = inputs.device_state((len(plens), H, d, d), 403, device=dev)
    dstate0 = inputs.device_state((B, H, d, d), 404, device=dev)
    dstate = dstate0.clone()
    pout, pfin = torch.empty_like(pq), torch.empty_like(pinit)
    dout = torch.empty_like(dq)
    # all twenty as one packed prefill (decode tokens as 1-token sequences)
    alens = plens + [1] * B
    acu = torch.from_numpy(inputs.cu_seqlens(alens)).to(dev)
    aq, ak, av = (torch.cat([x, y.transpose(0, 1)], dim=1).contiguous()
                  for x, y in ((pq, dq), (pk, dk), (pv, dv)))
    ainit = torch.cat([pinit, dstate0], dim=0).contiguous()
    aout, afin = torch.empty_like(aq), torch.empty_like(ainit)
    side = torch.cuda.Stream(device=dev)

    blk = [128]

    def prefill():
        la.lightning_attn_fwd_varlen(pq, pk, pv, decay, cu, init_states=pinit, out=pout,
                                     final_states=pfin, segment_tokens=seg, block=blk[0])

    def decode():
        la.lightning_attn_decode(dq, dk, dv, decay, dstate, out=dout)

    def serial():
        la.lightning_attn_mixed_step(decay, (pq, pk, pv), cu, (dq, dk, dv), dstate,
                                     init_states=pinit, prefill_out=pout, final_states=pfin,
                                     decode_out=dout, segment_tokens=seg)

    def two_streams():
        cur = torch.cuda.current_stream(dev)
        side.wait_stream(cur)
        la.lightning_attn_mixed_step(decay, (pq, pk, pv), cu, (dq, dk, dv), dstate,
                                     init_states=pinit, prefill_out=pout, final_states=pfin,
                                     decode_out=dout, segment_tokens=seg, decode_stream=side)
        cur.wait_stream(side)

    def one_varlen():
        la.lightning_attn_fwd_varlen(aq, ak, av, decay, acu, init_states=ainit, out=aout,
                                     final_states=afin, segment_tokens=seg, block=blk[0])

    res = {"workload": "serving_mix_h64", "H": H, "d": d,
           "batch": "2 sequences x %d new tokens + 18 x 1 token, all from prefix states" % P,
           "unit": "us per step"}
    variants = [("prefill_only", prefill, 128), ("decode_only", decode, 128),
                ("one_stream", serial, 128), ("two_streams", two_streams, 128),
                ("one_packed_prefill", one_varlen, 128)]
    # the short-chunk kernel (block 64 and 32) for the prefill parts
    for b in (64, 32):
        variants += [("prefill_only_block%d" % b, prefill, b),
                     ("one_packed_prefill_block%d" % b, one_varlen, b)]
    # the level the library picks from the mean input length (LA_BLOCK_AUTO)
    variants += [("prefill_only_block_auto", prefill, la.LA_BLOCK_AUTO),
                 ("one_packed_prefill_block_auto", one_varlen, la.LA_BLOCK_AUTO)]
    for name, fn, b in variants:
        blk[0] = b
        for _ in range(5):  # warm-up (and lazy initialisation) outside the capture
            fn()
        torch.cuda.synchronize()
        eager = []
        for _ in range(50):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            eager.append(s.elapsed_time(e) * 1e3)
        eager.sort()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(20):
            g.replay()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            g.replay()
        e.record()
        torch.cuda.synchronize()
        res[name] = {"eager": round(eager[len(eager) // 2], 2),
                     "graph": round(s.elapsed_time(e) * 1e3 / reps, 2)}
        del g
    blk[0] = 128
    dstate.copy_(dstate0)
    if P == 50:
        res["block_levels"] = bench_block_levels(la, inputs)
    return res


def bench_block_levels(la, inputs, S=32, reps=50):
    """Packed prefill of S equal sequences (64 heads, prefix states, one
    segment per sequence) at each block level, by sequence length: graph
    replays, microseconds per call.  The measurement behind the levels
    LA_BLOCK_AUTO picks from the mean length."""
    import torch
    dev = torch.device("cuda:0")
    H, d = 64, 128
    decay = torch.from_numpy(inputs.decay_schedule(H)).to(dev)
    init = inputs.device_state((S, H, d, d), 411, device=dev)
    fin = torch.empty_like(init)
    res = {"workload": "%d sequences x L tokens, H64, from prefix states" % S,
           "unit": "us per call (graph)"}
    for L in (8, 24, 32, 48, 64, 96, 128, 192):
        cu = torch.from_numpy(inputs.cu_seqlens([L] * S)).to(dev)
        q, k, v = inputs.device_qkv((H, S * L, d), 412 + L, "bf16", device=dev)
        out = torch.empty_like(q)
        row = {}
        for b in (32, 64, 128, la.LA_BLOCK_AUTO):
            def fn():
                la.lightning_attn_fwd_varlen(q, k, v, decay, cu, init_states=init, out=out,
                                             final_states=fin,
                                             segment_tokens=la.LA_SEGMENT_PER_SEQUENCE, block=b)
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            for _ in range(10):
                g.replay()
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                g.replay()
            e.record()
            torch.cuda.synchronize()
            row["auto" if b == la.LA_BLOCK_AUTO else str(b)] = round(
                s.elapsed_time(e) * 1e3 / reps, 2)
            del g
        res["L%d" % L] = row
    return res


def cpu_baseline(gpu_tensors, H, N, d, heads):
    """The oracle (untuned) on the host cores: `heads` of the H heads, all N
    tokens, on the same inputs; scaled to whole-workload tokens/s.  Also the
    parity of the timed run's own output and final state against it (the
    whole-tensor metric over the heads the oracle ran)."""
    import numpy as np
    import torch
    import oracle
    from linear_attention_lightning_amd import inputs
    q, k, v = (t[:, :heads].float().cpu().numpy() for t in gpu_tensors[:3])
    lam = inputs.decay_schedule(H)[:heads]
    t0 = time.perf_counter()
    o_ref, f_ref, used = oracle.fwd(q, k, v, lam)
    dt = time.perf_counter() - t0
    del q, k, v
    out, fin = gpu_tensors[4], gpu_tensors[5]
    num = den = 0.0
    for h in range(heads):
        a = out[:, h].float().cpu().numpy().astype(np.float64)
        if not np.isfinite(a).all():
            num = float("inf")
            break
        num = max(num, float(np.abs(a - o_ref[:, h]).max()))
        den = max(den, float(np.abs(o_ref[:, h]).max()))
    fs = fin[:, :heads].cpu().numpy().astype(np.float64)
    parity = {"out": num / den, "state": float(np.abs(fs - f_ref).max() / np.abs(f_ref).max()),
              "tolerance": 2e-2, "metric": "max|x - x_ref| / max|x_ref| over every element",
              "compared": "the last timed step's out and final_state, %d of %d heads, all %d "
                          "tokens, against the double-precision oracle" % (heads, H, N)}
    frac = heads / H
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(N / (dt / frac), 1), "unit": "tokens/s", "cores": used,
            "cpu_model": model, "kind": "oracle",
            "sample": "%d of %d heads, all %d tokens of the B=1 H=64 N=32768 d=128 workload "
                      "(double-precision recurrence), %.1f s wall; scaled to all heads"
                      % (heads, H, N, dt)}, parity


def copy_ceiling(mib=1024, reps=10):
    """A device-to-device torch copy of `mib` MiB, timed with HIP events:
    the practical ceiling of a 1:1 read/write stream on this GPU (median of
    `reps` copies; bytes read plus bytes written per second)."""
    import torch
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        dst.copy_(src)
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    times.sort()
    ms = times[len(times) // 2]
    gbs = 2 * (mib << 20) / (ms * 1e-3) / 1e9
    del src, dst
    return {"bytes_copied": mib << 20, "ms": round(ms, 4), "gbs_read_plus_write": round(gbs, 1),
            "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
            "note": "torch device copy, median of %d; the chunk kernel reads 3 bytes for each "
                    "byte it writes" % reps}


def run_metadata(seed):
    """Device, software versions and the input seed of this run."""
    import ctypes
    import torch
    p = torch.cuda.get_device_properties(0)
    md = {"device": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count,
          "hbm_bytes": p.total_memory, "torch": torch.__version__, "hip": torch.version.hip,
          "seed": seed, "timing": "HIP events on the library's stream"}
    try:
        with open("/opt/rocm/.info/version") as f:
            md["rocm"] = f.read().strip()
    except OSError:
        md["rocm"] = None
    try:
        # hipDeviceGetAttribute: 5 = clock rate, 60 = memory clock rate (kHz;
        # the peak figures the runtime reports, not the clock during the run)
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int()
        for name, attr in (("peak_sclk_mhz", 5), ("peak_mclk_mhz", 60)):
            md[name] = (v.value // 1000
                        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, 0) == 0 else None)
    except OSError:
        pass
    return md


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # After start-up the GPU's clock goes through a transient under
    # back-to-back work: the chunk kernel takes about 370 us in its first
    # launches, up to 530 us a few steps later, and recovers to 380-390 us
    # over the following tens of launches.  The default warm-up covers it;
    # with a short one (say 5 steps) the timed steps fall into the slow part,
    # and the steady_state object (the same step at the end of the run, after
    # a warm-up of its own) shows the settled figure beside it.
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=64)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, copy a buffer of this size once (a plain "
                         "copy kernel of known size, to scale HBM byte counters)")
    ap.add_argument("--trace", action="store_true",
                    help="also report the time of every headline step (warm-up and timed), "
                         "from HIP events between the steps")
    ap.add_argument("--leg", choices=["backward", "backward_varlen", "serving", "snapshots",
                                      "chdecay", "million", "varlen", "decode", "short_gated"],
                    default=None,
                    help="time only this extra workload and print its JSON object (for "
                         "profiling it on its own); the headline line is not printed")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: the library runs on one GPU only; --gpus %d is not supported "
              "(across GPUs, (batch, head) pairs or sequence segments would be sharded, "
              "each GPU running this path on its share)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_lightning_amd as la
    from linear_attention_lightning_amd import inputs

    la.load_library()
    if args.leg:
        legs = {"backward": lambda: bench_backward(la, inputs, args.steps, 20),
                "backward_varlen": lambda: bench_backward_varlen(la, inputs, args.steps, 5),
                "serving": lambda: bench_serving(la, inputs, P=50),
                "snapshots": lambda: bench_snapshots(la, inputs, args.steps, 2),
                "chdecay": lambda: bench_chdecay(la, inputs, args.steps, 20),
                "million": lambda: bench_million(la, inputs, args.steps, 2),
                "varlen": lambda: bench_varlen(la, inputs, args.steps, 2),
                "decode": lambda: bench_decode(la, inputs, reps=5, warmup=1),
                "short_gated": lambda: bench_short_gated(la, inputs, args.steps, 20)}
        print(json.dumps(legs[args.leg]()), flush=True)
        return
    w = inputs.WORKLOADS["layer_h64_n32k"]
    B, H, N, d, block = w["B"], w["H"], w["N"], w["d"], w["block"]
    trace = [] if args.trace else None
    ms, phase_ms, tensors = bench_prefill(la, inputs, B, H, N, d, block, w["seed"], args.steps,
                                          args.warmup, phases=True, trace=trace)
    sec = ms * 1e-3
    flops = prefill_flops(B, H, N, d, block)
    tflops = flops / sec / 1e12
    alg = prefill_bytes(B, H, N, d)
    gbs = alg / sec / 1e9
    traffic = measured_traffic("layer_h64_n32k") or {}
    # The dominant kernel is the output pass (prefill_chunk_kernel): it reads
    # q, k, v and writes out and the final states, i.e. the path's algorithmic
    # bytes, once per launch.
    chunk_s = phase_ms[2] * 1e-3
    chunk_gbs = alg / chunk_s / 1e9
    res = {
        "metric": METRIC,
        "value": round(B * N / sec, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "layer_h64_n32k", "B": B, "H": H, "N": N, "d": d,
                   "block": block, "state": "fp32"},
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(chunk_gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(chunk_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic.get("prefill_chunk_kernel"),
                     "kernel": "la::mfma::prefill_chunk_kernel",
                     "launch_us": round(phase_ms[2] * 1e3, 1),
                     "algorithmic_bytes_per_launch": alg},
        "phases_us": {"sampled_steps": max(1, args.steps // 5),
                      "local_state_kernel": round(phase_ms[0] * 1e3, 1),
                      "segment_scan_kernel": round(phase_ms[1] * 1e3, 1),
                      "prefill_chunk_kernel": round(phase_ms[2] * 1e3, 1)},
        "step_hbm": {"achieved": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic.get("step"), "unit": "GB/s",
                     "note": "algorithmic bytes per step / step time; traffic = counter "
                             "bytes of all three kernels per step"},
    }
    if trace is not None:
        res["per_step_us"] = trace
    res["run"] = run_metadata(w["seed"])
    res["copy_ceiling"] = copy_ceiling()
    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = nbytes
        del src, dst
    if not args.no_cpu_baseline:
        res["cpu_baseline"], res["parity"] = cpu_baseline(tensors, H, N, d, min(args.cpu_heads, H))
    del tensors
    torch.cuda.empty_cache()
    if not args.no_extras:
        res["decode"] = bench_decode(la, inputs, reps=5, warmup=1)
        torch.cuda.empty_cache()
        res["varlen"] = bench_varlen(la, inputs, steps=max(5, args.steps // 2), warmup=2)
        torch.cuda.empty_cache()
        res["million"] = bench_million(la, inputs, steps=5, warmup=1)
        torch.cuda.empty_cache()
        res["token_major"] = bench_token_major(la, inputs, steps=args.steps, warmup=args.warmup)
        torch.cuda.empty_cache()
        res["backward"] = bench_backward(la, inputs, steps=args.steps, warmup=20)
        torch.cuda.empty_cache()
        res["backward_varlen"] = bench_backward_varlen(la, inputs, steps=max(5, args.steps // 2),
                                                       warmup=5)
        torch.cuda.empty_cache()
        res["chdecay"] = bench_chdecay(la, inputs, steps=args.steps, warmup=20)
        torch.cuda.empty_cache()
        res["snapshots"] = bench_snapshots(la, inputs, steps=max(5, args.steps // 2), warmup=2)
        torch.cuda.empty_cache()
        res["short_gated"] = bench_short_gated(la, inputs, steps=args.steps, warmup=20)
        torch.cuda.empty_cache()
        res["serving"] = bench_serving(la, inputs, P=50)
        torch.cuda.empty_cache()
        res["serving_long"] = bench_serving(la, inputs, P=2048)
        torch.cuda.empty_cache()
        res["steady_state"] = bench_steady(la, inputs, w, args.steps)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
