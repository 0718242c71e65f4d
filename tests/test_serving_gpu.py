"""GPU parity of the serving-side entry points against the CPU oracle:
prefix-state snapshots of packed prefill (a prefix cache for linear
attention: K3 reading notes, inference-engine part, one prefix state per
block; MiniMax-01 report, sections 3.3.2-3.3.3, batches whose inputs carry a
prefix cache) and continuation from them.

Bar as in test_parity_gpu.py: max |x - x_ref| / max |x_ref| <= 1e-4 for
float32 inputs, <= 2e-2 for bf16 inputs, for outputs, final states and
snapshots; every snapshot row is checked to be written (buffers start as NaN).
"""
import sys

import numpy as np
import pytest

import oracle
import linear_attention_lightning_amd as la
from linear_attention_lightning_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}

LENS = [300, 0, 1, 129, 1024, 5, 0, 640, 2000, 256, 97]


@pytest.fixture(params=["auto", "phased", "fused"])
def prefill_path(request, monkeypatch):
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
    den = np.abs(b).max() if b.size else 0.0
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0)) if a.size else 0.0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    torch = torch_mod()
    return t.detach().to(torch.float32).cpu().numpy()


def dev_inputs(shape, seed, dtype):
    torch = torch_mod()
    q, k, v = inputs.host_qkv(shape, seed, dtype=dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return [torch.from_numpy(x).to("cuda").to(tdt) for x in (q, k, v)], (q, k, v)


def run_snapshot_case(lens, H, d, dtype, seed, iv, seg=0, with_init=True, token_major=False):
    torch = torch_mod()
    say("case snapshots lens=%s H=%d d=%d %s iv=%d seg=%d token_major=%s"
        % (lens[:8], H, d, dtype, iv, seg, token_major))
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    (tq, tk, tv), (q, k, v) = dev_inputs((H, total, d), seed, dtype)
    lam = inputs.decay_schedule(H)
    init = inputs.host_state((len(lens), H, d, d), seed + 1) if with_init else None
    ti = torch.from_numpy(init).cuda() if with_init else None
    tcu = torch.from_numpy(cu).cuda()
    offs = la.snapshot_row_offsets(tcu, iv)
    snaps = torch.full((offs[-1], H, d, d), float("nan"), device="cuda")
    layout = la.LA_HEAD_MAJOR
    if token_major:
        tq, tk, tv = (t.transpose(0, 1).contiguous() for t in (tq, tk, tv))  # [total, H, d]
        layout = la.LA_TOKEN_MAJOR
    out = torch.full_like(tq, float("nan"))
    out, fin, snaps, toffs = la.lightning_attn_fwd_varlen_snapshots(
        tq, tk, tv, torch.from_numpy(lam).cuda(), tcu, iv, layout=layout, init_states=ti,
        segment_tokens=seg, out=out, snapshots=snaps)
    torch.cuda.synchronize()
    if token_major:
        out = out.transpose(0, 1)
    o_ref, f_ref, s_ref, offs_ref = oracle.fwd_varlen_snapshots(q, k, v, lam, cu, iv, init=init)
    assert list(offs_ref) == offs and toffs.tolist() == offs
    so = host(snaps)
    assert np.isfinite(so).all(), "a snapshot row was not written"
    assert bool(torch.isfinite(out).all())
    eo = rel_err(host(out), o_ref) if total else 0.0
    ef, es = rel_err(host(fin), f_ref), rel_err(so, s_ref)
    say("   %d snapshot rows; err out %.3e state %.3e snapshots %.3e" % (offs[-1], eo, ef, es))
    assert eo <= TOL[dtype] and ef <= TOL[dtype] and es <= TOL[dtype], (eo, ef, es)


@pytest.mark.parametrize("iv", [128, 256, 96, 1000])
@pytest.mark.parametrize("seg", [0, 200, 1000, la.LA_SEGMENT_PER_SEQUENCE])
def test_snapshots_bf16(iv, seg, prefill_path):
    """Snapshot intervals that are multiples of the 128-token chunk and ones
    that are not (96, 1000), with segments that start inside sequences at
    offsets off the snapshot grid (200, 1000): chunks are cut at every
    snapshot point, and the state there is stored."""
    run_snapshot_case(LENS, 4, 128, "bf16", seed=200 + iv + seg, iv=iv, seg=seg)


def test_snapshots_short_interval():
    """16-token snapshots: chunks of 16 tokens throughout."""
    run_snapshot_case([300, 0, 1, 129, 64], 3, 128, "bf16", seed=210, iv=16, seg=100)


@pytest.mark.parametrize("seg", [0, 200])
def test_snapshots_token_major(seg, prefill_path):
    run_snapshot_case(LENS, 4, 128, "bf16", seed=220 + seg, iv=128, seg=seg, token_major=True)


@pytest.mark.parametrize("d,dtype,iv", [(64, "fp32", 32), (128, "fp32", 50), (64, "bf16", 64)])
@pytest.mark.parametrize("seg", [0, 48, la.LA_SEGMENT_PER_SEQUENCE])
def test_snapshots_vector_alu(d, dtype, iv, seg):
    run_snapshot_case([33, 0, 64, 1, 100, 160], 2, d, dtype, seed=230 + d + iv, iv=iv, seg=seg)


def test_snapshots_without_initial_state():
    run_snapshot_case(LENS, 4, 128, "bf16", seed=240, iv=128, with_init=False)


def test_no_snapshot_due():
    """An interval longer than every sequence stores nothing and leaves the
    prefill's results unchanged."""
    run_snapshot_case([5, 0, 7, 30], 2, 128, "bf16", seed=250, iv=100)
    run_snapshot_case([5, 7], 2, 128, "bf16", seed=251, iv=13)  # total 12 < 13


def test_continue_from_snapshot():
    """Prefix caching: a request that shares the first m * 256 tokens of a
    prefilled sequence starts from snapshot m and prefills only the rest; its
    outputs and final state are the full sequence's (oracle)."""
    torch = torch_mod()
    H, d, iv = 4, 128, 256
    lens = [3000, 1500]
    say("case continue from snapshot lens=%s iv=%d" % (lens, iv))
    cu = inputs.cu_seqlens(lens)
    (tq, tk, tv), (q, k, v) = dev_inputs((H, int(cu[-1]), d), 260, "bf16")
    lam = inputs.decay_schedule(H)
    tl = torch.from_numpy(lam).cuda()
    _, _, snaps, offs = la.lightning_attn_fwd_varlen_snapshots(
        tq, tk, tv, tl, torch.from_numpy(cu).cuda(), iv)
    o_ref, f_ref, _ = oracle.fwd_varlen(q, k, v, lam, cu)
    offs = offs.tolist()
    for j, m in ((0, 5), (0, 11), (1, 1), (1, 5)):
        a, b = int(cu[j]) + m * iv, int(cu[j + 1])
        sub = [t[:, a:b].contiguous() for t in (tq, tk, tv)]
        init = snaps[offs[j] + m - 1][None].contiguous()
        out, fin = la.lightning_attn_fwd_varlen(
            *sub, tl, torch.tensor([0, b - a], dtype=torch.int32, device="cuda"),
            init_states=init)
        torch.cuda.synchronize()
        eo = rel_err(host(out), o_ref[:, a:b])
        ef = rel_err(host(fin[0]), f_ref[j])
        say("   seq %d from snapshot %d: err out %.3e state %.3e" % (j, m, eo, ef))
        assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


def test_full_varlen_h64_65536_snapshots():
    """The 65536-token packed workload (lognormal lengths, H = 64) with a
    snapshot every 256 tokens, in the launch configuration the benchmark
    times: sampled snapshot entries against the oracle's closed-form prefix
    state, every row written, and whole sequences' outputs unchanged in
    accuracy."""
    torch = torch_mod()
    w = inputs.WORKLOADS["layer_h64_varlen64k"]
    H, total, d, iv = w["H"], w["total"], w["d"], 256
    lens = inputs.varlen_lengths(total=total, seed=w["seed"])
    cu = inputs.cu_seqlens(lens)
    say("case full varlen snapshots: %d sequences, interval %d" % (len(lens), iv))
    tq, tk, tv = inputs.device_qkv((H, total, d), w["seed"], "bf16")
    lam = inputs.decay_schedule(H)
    tcu = torch.from_numpy(cu).cuda()
    offs = la.snapshot_row_offsets(tcu, iv)
    snaps = torch.full((offs[-1], H, d, d), float("nan"), device="cuda")
    out, fin, snaps, _ = la.lightning_attn_fwd_varlen_snapshots(
        tq, tk, tv, torch.from_numpy(lam).cuda(), tcu, iv, block=w["block"], snapshots=snaps)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(snaps).all())
    rng = np.random.default_rng(3)
    ij = rng.integers(0, d, (16, 2))
    j_long = int(np.argmax(lens))
    picks = [(j_long, 1), (j_long, lens[j_long] // iv), (0, max(lens[0] // iv, 1))]
    worst = 0.0
    for j, m in picks:
        if m > lens[j] // iv:
            continue
        a = int(cu[j])
        for h in (0, 17, H - 1):
            kh, vh = (host(t[h, a:a + m * iv]) for t in (tk, tv))
            ref = oracle.state_entries(kh, vh, lam[h], ij)
            got = host(snaps[offs[j] + m - 1, h])[ij[:, 0], ij[:, 1]]
            worst = max(worst, rel_err(got, ref))
    say("   %d snapshot rows; worst sampled err %.3e" % (offs[-1], worst))
    assert worst <= TOL["bf16"]
    a, b = int(cu[j_long]), int(cu[j_long + 1])
    for h in (0, H - 1):
        qh, kh, vh = (host(t[h:h + 1, a:b])[None] for t in (tq, tk, tv))
        o_ref, f_ref, _ = oracle.fwd(qh, kh, vh, lam[h:h + 1])
        eo = rel_err(host(out[h, a:b]), o_ref[0, 0])
        ef = rel_err(host(fin[j_long, h]), f_ref[0, 0])
        say("   longest sequence, head %d: err out %.3e state %.3e" % (h, eo, ef))
        assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
    # the last snapshot of a sequence whose length is a multiple of the
    # interval equals its final state
    for j, n in enumerate(lens):
        if n and n % iv == 0:
            assert torch.equal(snaps[offs[j + 1] - 1], fin[j])


# ------------------------------------------------------- mixed serving step


def run_mixed_case(prefill_lens, decode_B, H, d, dtype, seed, two_streams=True,
                   token_major=False, seg=0, block=128):
    """Sequences with prefix states: the prefill part continues len > 1
    prompts from their prefix states, the decode part takes one token for
    each of decode_B others; both against the oracle (packed recurrence from
    the prefix state; recurrent decode step)."""
    torch = torch_mod()
    say("case mixed prefill=%s decode_B=%d H=%d d=%d %s two_streams=%s token_major=%s seg=%d"
        % (prefill_lens, decode_B, H, d, dtype, two_streams, token_major, seg))
    cu = inputs.cu_seqlens(prefill_lens)
    total = int(cu[-1])
    (pq, pk, pv), (hq, hk, hv) = dev_inputs((H, total, d), seed, dtype)
    (dq, dk, dv), (eq, ek, ev) = dev_inputs((decode_B, H, d), seed + 1, dtype)
    lam = inputs.decay_schedule(H)
    tl = torch.from_numpy(lam).cuda()
    P0 = inputs.host_state((len(prefill_lens), H, d, d), seed + 2)
    D0 = inputs.host_state((decode_B, H, d, d), seed + 3)
    dstate = torch.from_numpy(D0).cuda()
    layout = la.LA_HEAD_MAJOR
    if token_major:
        pq, pk, pv = (t.transpose(0, 1).contiguous() for t in (pq, pk, pv))
        layout = la.LA_TOKEN_MAJOR
    side = torch.cuda.Stream() if two_streams else None
    torch.cuda.synchronize()
    pout, fin, dout = la.lightning_attn_mixed_step(
        tl, (pq, pk, pv), torch.from_numpy(cu).cuda(), (dq, dk, dv), dstate, layout=layout,
        init_states=torch.from_numpy(P0).cuda(), decode_stream=side, segment_tokens=seg,
        block=block)
    torch.cuda.synchronize()
    if token_major:
        pout = pout.transpose(0, 1)
    o_ref, f_ref, _ = oracle.fwd_varlen(hq, hk, hv, lam, cu, init=P0)
    S = D0.astype(np.float64)
    d_ref, _ = oracle.decode(eq, ek, ev, lam, S)
    eo = rel_err(host(pout), o_ref) if total else 0.0
    ef = rel_err(host(fin), f_ref) if len(prefill_lens) else 0.0
    ed = rel_err(host(dout), d_ref) if decode_B else 0.0
    es = rel_err(host(dstate), S) if decode_B else 0.0
    say("   err prefill out %.3e state %.3e; decode out %.3e state %.3e" % (eo, ef, ed, es))
    assert max(eo, ef, ed, es) <= TOL[dtype], (eo, ef, ed, es)


@pytest.mark.parametrize("two_streams", [True, False])
@pytest.mark.parametrize("seg", [0, la.LA_SEGMENT_PER_SEQUENCE])
def test_mixed_step_pages_scenario(two_streams, seg):
    """Batch of 20 with prefix states: two inputs of 50 tokens, eighteen of
    one token (the mix of MiniMax-01 report section 3.3.2), at the 64-head
    layer shape."""
    run_mixed_case([50, 50], 18, 64, 128, "bf16", seed=300, two_streams=two_streams, seg=seg)


@pytest.mark.parametrize("two_streams", [True, False])
def test_mixed_step_block_auto(two_streams):
    """The pages' mix with the prefill part's block level picked from its mean
    length (LA_BLOCK_AUTO: 2 x 50 tokens -> block 64), and a mix of longer
    continuations (mean 300 -> block 128)."""
    run_mixed_case([50, 50], 18, 64, 128, "bf16", seed=305, two_streams=two_streams,
                   seg=la.LA_SEGMENT_PER_SEQUENCE, block=la.LA_BLOCK_AUTO)
    run_mixed_case([300, 1, 599], 9, 8, 128, "bf16", seed=306, two_streams=two_streams,
                   block=la.LA_BLOCK_AUTO)


@pytest.mark.parametrize("d,dtype", [(64, "fp32"), (128, "fp32"), (64, "bf16")])
def test_mixed_step_vector_alu(d, dtype):
    run_mixed_case([7, 0, 40], 5, 4, d, dtype, seed=310 + d)
    run_mixed_case([7, 0, 40], 5, 4, d, dtype, seed=311 + d, seg=la.LA_SEGMENT_PER_SEQUENCE)


def test_mixed_step_token_major():
    run_mixed_case([300, 1, 129], 9, 8, 128, "bf16", seed=320, token_major=True)


def test_mixed_step_one_part_empty():
    run_mixed_case([], 6, 8, 128, "bf16", seed=330)
    run_mixed_case([64, 200], 0, 8, 128, "bf16", seed=331)


def test_mixed_step_graph_replay():
    """The two-stream step captured as a HIP graph (as a serving loop would
    run it) gives the eager step's results, bit for bit, on every replay;
    eager work and synchronisations run between the replays."""
    torch = torch_mod()
    H, d, B = 16, 128, 6
    plens = [50, 50, 3]
    say("case mixed step graph replay")
    cu = torch.from_numpy(inputs.cu_seqlens(plens)).cuda()
    (pq, pk, pv), _ = dev_inputs((H, sum(plens), d), 340, "bf16")
    (dq, dk, dv), _ = dev_inputs((B, H, d), 341, "bf16")
    tl = torch.from_numpy(inputs.decay_schedule(H)).cuda()
    pinit = torch.from_numpy(inputs.host_state((len(plens), H, d, d), 342)).cuda()
    D0 = torch.from_numpy(inputs.host_state((B, H, d, d), 343)).cuda()
    dstate = D0.clone()
    pout, pfin, dout = torch.empty_like(pq), torch.empty_like(pinit), torch.empty_like(dq)
    nws = la.lightning_attn_fwd_varlen_workspace_size(len(plens), H, sum(plens), d, 128)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()

    def step():
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        la.lightning_attn_mixed_step(tl, (pq, pk, pv), cu, (dq, dk, dv), dstate,
                                     init_states=pinit, prefill_out=pout, final_states=pfin,
                                     decode_out=dout, workspace=ws, decode_stream=side)
        cur.wait_stream(side)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (pout, pfin, dout, dstate)]
    g = torch.cuda.CUDAGraph()
    dstate.copy_(D0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        for t in (pout, pfin, dout):
            t.fill_(float("nan"))
        dstate.copy_(D0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("prefill out", "final states", "decode out", "state"),
                                   (pout, pfin, dout, dstate), ref):
            assert torch.equal(got, want), "replay %d: %s differs" % (r, name)
