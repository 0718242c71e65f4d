"""Phase timing of the 128-token chunk kernel, from the shader clock.

    python -m linear_attention_lightning_amd.phase_probe --build     # CPU: instrumented build
    python -m linear_attention_lightning_amd.phase_probe [--warmup W] [--json FILE]   # GPU

The build compiles the library's sources with -DLA_PHASE_PROBE into
_build/liblightning_attn_phase_probe.so (the library proper is unchanged:
without the macro the marks compile to nothing).  In that build, lane 0 of
output wave 0 and of state wave 4 of each of the first 256 workgroups
records s_memtime at the barriers and phase ends of its first 64 chunks.
The run does W prefill steps of the B=1 H=64 N=32768 d=128 bf16 workload
(4 segments of 8192 tokens per head: 256 workgroups, 64 chunks each), clears
the record, runs one more step and prints, per phase, the median and 10th /
90th percentiles over workgroups and chunks (the first and last chunk of each
walk left out) in shader-clock cycles.

The local-state pass (first 1024 workgroups, first 40 of its 64-token chunks, thread 0) is
recorded in the same step: chunk start -> tiles stored and first barrier -> state update ->
second barrier.

Phases of the chunk kernel (one chunk, between barrier A that opens it and the next chunk's A):
  output wave: A -> inter-block term done -> steps shared by both query
  blocks done -> remaining steps done -> B -> rows staged and written -> A
  state wave:  A -> state update done -> B -> S^T published -> next tiles
  landed -> A
"""
import argparse
import ctypes
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROBE_LIB = os.path.join(ROOT, "_build", "liblightning_attn_phase_probe.so")

OUT_PHASES = [(0, 1, "out: A -> inter-block term"),
              (1, 2, "out: -> shared key steps (both blocks)"),
              (2, 3, "out: -> remaining key steps (block 7-w)"),
              (3, 4, "out: -> barrier B passed"),
              (4, 5, "out: -> rows staged and written")]
LOCAL_PHASES = [(0, 1, "local: chunk start -> tiles stored, barrier"),
                (1, 2, "local: -> state update"),
                (2, 3, "local: -> second barrier")]
STATE_PHASES = [(8, 9, "state: A -> state update"),
                (9, 10, "state: -> barrier B passed"),
                (10, 11, "state: -> S^T published"),
                (11, 12, "state: -> next tiles landed")]


def build():
    from . import build as b
    os.makedirs(os.path.dirname(PROBE_LIB), exist_ok=True)
    return b.build(out=PROBE_LIB, extra=["-DLA_PHASE_PROBE"])


def run(warmup):
    import numpy as np
    import torch
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError("%s is not built; run with --build first (on the host)" % PROBE_LIB)
    # every call of the binding below goes through the instrumented build
    os.environ["LIGHTNING_ATTN_LIB"] = PROBE_LIB
    import linear_attention_lightning_amd as la
    from . import inputs
    lib = la.load_library()
    if not hasattr(lib, "lightning_attn_phase_probe_copy"):
        raise RuntimeError("the binding had already loaded another library")
    lib.lightning_attn_phase_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.lightning_attn_phase_probe_copy_local.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    B, H, N, d = 1, 64, 32768, 128
    dev = torch.device("cuda:0")
    q, k, v = inputs.device_qkv((B, H, N, d), 3, "bf16", device=dev)
    lam = torch.from_numpy(inputs.decay_schedule(H)).to(dev)
    out = torch.empty_like(q)
    fin = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    ws = torch.empty(la.lightning_attn_fwd_workspace_size(B, H, N, d, 128), dtype=torch.uint8,
                     device=dev)

    def step():
        la.lightning_attn_fwd(q, k, v, lam, block=128, out=out, final_state=fin, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if lib.lightning_attn_phase_probe_clear() != 0:
        raise RuntimeError("phase record could not be cleared")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    step()
    e1.record()
    torch.cuda.synchronize()
    rec = np.zeros(256 * 64 * 16, np.uint64)
    if lib.lightning_attn_phase_probe_copy(rec.ctypes.data, rec.nbytes) != 0:
        raise RuntimeError("phase record could not be read")
    P = rec.reshape(256, 64, 16).astype(np.int64)
    # (the state waves leave the walk at the last chunk's barrier B: no
    # publish or tile wait there)
    if not ((P[:, :, [0, 1, 2, 3, 4, 5, 8, 9, 10]] > 0).all() and (P[:, :63, [11, 12]] > 0).all()):
        raise RuntimeError("incomplete phase record (plan not 256 workgroups x 64 chunks?)")

    def stats(x):
        x = np.asarray(x).ravel()
        return {"median": float(np.median(x)), "p10": float(np.percentile(x, 10)),
                "p90": float(np.percentile(x, 90))}

    res = {"workload": "layer_h64_n32k", "warmup_steps": warmup, "step_ms": e0.elapsed_time(e1),
           "unit": "shader-clock cycles per chunk", "phases": {}}
    mid = slice(1, 63)
    for a, b, name in OUT_PHASES + STATE_PHASES:
        res["phases"][name] = stats(P[:, mid, b] - P[:, mid, a])
    res["phases"]["out: rows written -> next A"] = stats(P[:, 2:63, 0] - P[:, 1:62, 5])
    res["phases"]["state: tiles landed -> next A"] = stats(P[:, 2:63, 8] - P[:, 1:62, 12])
    res["phases"]["chunk period (A to A)"] = stats(P[:, 2:63, 0] - P[:, 1:62, 0])
    res["workgroup_walk_cycles"] = stats(P[:, 63, 5] - P[:, 0, 0])
    # the local-state pass: workgroups with at least three chunks, chunks from the second on
    loc = np.zeros(1024 * 40 * 4, np.uint64)
    if lib.lightning_attn_phase_probe_copy_local(loc.ctypes.data, loc.nbytes) != 0:
        raise RuntimeError("local-pass phase record could not be read")
    Q = loc.reshape(1024, 40, 4).astype(np.int64)
    nch = (Q[:, :, 3] > 0).sum(1)
    sel = [(w, c) for w in range(1024) for c in range(1, nch[w]) if nch[w] >= 3]
    lp = {}
    for a, b, name in LOCAL_PHASES:
        lp[name] = stats([Q[w, c, b] - Q[w, c, a] for w, c in sel])
    lp["chunk period"] = stats([Q[w, c, 0] - Q[w, c - 1, 0] for w, c in sel])
    full = [w for w in range(1024) if nch[w] == nch.max()]
    res["local_pass"] = {"workgroups_with_work": int((nch > 0).sum()),
                         "chunks_per_workgroup_max": int(nch.max()),
                         "workgroups_at_max": len(full),
                         "walk_cycles_at_max": stats([Q[w, nch[w] - 1, 3] - Q[w, 0, 0] for w in full]),
                         "phases": lp}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--build", action="store_true", help="build the instrumented library and exit")
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--json", default=None, help="also write the result here")
    args = ap.parse_args()
    if args.build:
        print(build())
        return
    res = run(args.warmup)
    print("step %.4f ms after %d warm-up steps; %s" % (res["step_ms"], args.warmup, res["unit"]))
    for name, st in res["phases"].items():
        print("%-44s median %7.0f   p10 %7.0f   p90 %7.0f" % (name, st["median"], st["p10"],
                                                                st["p90"]))
    st = res["workgroup_walk_cycles"]
    print("%-44s median %7.0f   p10 %7.0f   p90 %7.0f" % ("whole walk of a workgroup", st["median"],
                                                            st["p10"], st["p90"]))
    lp = res["local_pass"]
    print("local-state pass: %d workgroups with work, %d walk the most chunks (%d), median walk %.0f cycles"
          % (lp["workgroups_with_work"], lp["workgroups_at_max"], lp["chunks_per_workgroup_max"],
             lp["walk_cycles_at_max"]["median"]))
    for name, st in lp["phases"].items():
        print("%-44s median %7.0f   p10 %7.0f   p90 %7.0f" % (name, st["median"], st["p10"],
                                                                st["p90"]))
    if args.json:
        with open(args.json, "w") as f:
            json.dump(res, f, indent=1)
    sys.stdout.flush()


if __name__ == "__main__":
    main()
