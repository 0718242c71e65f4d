// Host side of the lightning attention library: argument checks, the
// segment plan, kernel launches and the exported C ABI (lightning_attn.h).
#include "lightning_attn.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "la_common.h"
#include "la_prefill_mfma.h"
#include "la_prefill_short.h"
#include "la_prefill_chdecay.h"
#include "la_prefill_simt.h"
#include "la_scan_decode.h"
#include "la_backward.h"

namespace {

using la::bf16;

constexpr int kVersion = 100;    // 0.1.0

bool valid_block(int b) {
  return b == LA_BLOCK_AUTO || b == 16 || b == 32 || b == 64 || b == 128 || b == 256;
}

// LA_BLOCK_AUTO: the block level from the call's mean input length (the
// MiniMax-01 report's multi-level padding, section 3.3.3, pads each input
// to the smallest of 32, 64, 128, 256 tokens that holds it).  Levels of 128
// and 256 run the same kernel, so 128 stands for both.
int level_block(int block, int64_t mean_len) {
  if (block != LA_BLOCK_AUTO) return block;
  return mean_len <= 32 ? 32 : mean_len <= 64 ? 64 : 128;
}
bool valid_d(int d) { return d == 64 || d == 128; }
bool valid_dtype(la_dtype dt) { return dt == LA_FP32 || dt == LA_BF16; }

// bf16 with d = 128 runs on MFMA; everything else on the vector ALUs.
// ch: the channel-wise decay variant (its own MFMA output pass, 64-token
// chunks; the vector-ALU kernels otherwise).
bool use_mfma(int d, la_dtype dt, bool ch = false) { (void)ch; return dt == LA_BF16 && d == 128; }
int chunk_tokens(int d, la_dtype dt, bool ch = false) {
  return use_mfma(d, dt, ch) ? (ch ? la::mfma::TC : la::mfma::T) : la::simt::T;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
  int64_t seg;   // segment length (tokens)
  int64_t nseg;  // segments per head
  bool scan;     // segments must hand states on (a scan is needed)
  bool fused;    // single-pass kernel hands states on itself (else 3 phases)
  int r_split;   // pieces per segment of the local-state pass
  size_t ws_bytes;
  int chunk;     // tokens per chunk of the output pass (bf16 MFMA: 128, or 64 / 32
                 // on the short-chunk kernel)
};

// Chunk of the output pass.  bf16 with d = 128 walks 128-token chunks on
// the MFMA kernel that takes a whole CU per workgroup; a forward prefill
// (short_ok) whose block is at most 64 tokens walks 64- or 32-token chunks
// on the short-chunk kernel instead, two workgroups per CU (the MiniMax-01
// report's multi-level padding to 32/64/128/256 tokens by input length,
// section 3.3.3, with the block length as the level: short inputs do not pay
// for a long block).  The backward, prefix snapshots and the channel-wise
// variant keep their own chunks.
int out_chunk(int d, la_dtype dt, bool ch, int block, bool short_ok) {
  if (short_ok && !ch && use_mfma(d, dt) && block <= 64) return block <= 32 ? 32 : 64;
  return chunk_tokens(d, dt, ch);
}

size_t state_bytes(int64_t count, int d) { return (size_t)count * (size_t)d * (size_t)d * 4; }

// Workspace of the single-pass kernel: end-state records, then one flag per
// (segment, head), a ticket counter and an error word.
size_t fused_ws_bytes(int64_t nseg, int H, int d) {
  return state_bytes(nseg * H, d) + (size_t)(nseg * H + 2) * 4;
}

// Prefill path.  The three-phase path (local states, scan, outputs) is the
// default.  The single-pass kernel (hand-offs between segments through the
// workspace, K/V re-reads from the Infinity Cache) moves a third less HBM
// traffic but serialises each workgroup's local-state pass, hand-off and
// outputs; on MI355X it measured slower than the default (604 against 541 us
// per step at B1 H64 N32768 with 8192-token segments), so it is opt-in:
// LIGHTNING_ATTN_PREFILL=fused selects it (MFMA path only), =phased forces
// the default.  Results agree up to rounding.
bool want_fused(int H, int d, la_dtype dt, bool ch = false) {
  (void)H;
  if (ch || !use_mfma(d, dt, ch)) return false;
  const char *e = getenv("LIGHTNING_ATTN_PREFILL");
  return e && strcmp(e, "fused") == 0;
}

// Segment length of the single-pass kernel: one round of 256 resident
// workgroups at the 64-head layer shape (fewest hand-offs), while the K/V of
// a round (256 x seg x 512 B) mostly stay in the 256 MB Infinity Cache.
constexpr int64_t kFusedSeg = 8192;

// Fixed-length plan.  Without a scan each sequence is one segment.  With
// one, the token axis of every head is cut into equal segments so that
// about target_groups(d, dt) workgroups run per phase.
// Workgroups to aim for per phase: the MFMA chunk kernel (160 KB of LDS) and
// the channel-wise one (82 KB) run one workgroup per CU, and a single round
// over the 256 CUs with long segments measured fastest (fewer, longer
// pipelines and less local-state work: for the channel-wise kernel 4
// segments per head instead of 8 took its 64-head 32768-token step from
// 770 to 716 us); the short-chunk kernel (two per CU) and the vector-ALU
// kernels run several workgroups per CU.
int64_t target_groups(int d, la_dtype dt, bool ch = false, int chunk = 128) {
  return use_mfma(d, dt, ch) && (chunk == la::mfma::T || ch) ? 256 : 512;
}

// Pieces per segment of the MFMA local-state pass (for a head whose whole
// segment carries weight; piece_plan gives a faster-decaying head fewer):
// 4 pieces of at least 8 chunks of 64 tokens for segments up to 8192 tokens,
// so that several workgroups share a CU and hide one another's latency (8 or
// 16 there made the pass faster but the scan, which reads every piece's
// partial state, slower by more); longer segments keep the pieces at 2048
// tokens, up to 16, since a piece is walked serially by one workgroup (at
// the 1M-token 8-head shape four 8192-token pieces per segment left the
// slowest heads' workgroups walking 128 chunks each).  A power of two (the
// pieces are cut by shifts).  The vector-ALU pass uses one.
int pieces(int64_t seg, int d, la_dtype dt, bool ch = false) {
  if (!use_mfma(d, dt, ch)) return 1;
  const int64_t r = seg / la::mfma::C_LOCAL / 8;
  int n = r >= 4 ? 4 : r >= 2 ? 2 : 1;
  while (n < 16 && (int64_t)n * 2048 < seg) n *= 2;
  return n;
}

// A launch holds at most 2^32 - 1 work-items (workgroups times their
// threads).  The widest grids of a plan: one workgroup of up to 512 threads
// per (segment, head) in the output pass, and r_split workgroups of 256
// threads per (segment, head) in the local-state pass.  Plans beyond that are
// refused before anything is launched.
bool plan_fits(const Plan &p, int H) {
  const int64_t groups = p.nseg * (int64_t)H;
  const int64_t lim = (int64_t)0xffffffff;
  return groups <= lim / 512 && groups <= lim / 256 / (p.r_split > 0 ? p.r_split : 1);
}

size_t phased_ws_bytes(const Plan &p, int H, int d) {
  return state_bytes(p.nseg * p.r_split * H, d);
}

// segment_tokens value: every sequence is one segment (see lightning_attn.h).
constexpr int64_t kSegPerSeq = -1;

Plan plan_fixed(int B, int H, int64_t N, int d, la_dtype dt, int64_t segment_tokens,
                bool allow_fused = true, bool ch = false, int block = 128,
                bool short_ok = false) {
  if (segment_tokens == kSegPerSeq) segment_tokens = N;  // N == 0: automatic (nothing to cut)
  const int T = out_chunk(d, dt, ch, level_block(block, N), short_ok);
  Plan p{N, B, false, false, 1, 0, T};
  const int64_t total = (int64_t)B * N;
  if (total == 0) {
    p.nseg = 0;
    return p;
  }
  int64_t seg = N;
  if (segment_tokens > 0) {
    seg = segment_tokens;
  } else {
    const int64_t bh = (int64_t)B * H;
    int64_t G = ceil_div(target_groups(d, dt, ch, T), bh);
    const int64_t maxG = ceil_div(N, T);
    if (G > maxG) G = maxG;
    if (G > 1) {
      seg = ceil_div(ceil_div(N, G), T) * T;
      if (seg >= N) seg = N;
    }
  }
  const bool fused = allow_fused && T == la::mfma::T && want_fused(H, d, dt, ch);
  if (fused && segment_tokens <= 0 && seg != N && seg > kFusedSeg) seg = kFusedSeg;
  p.seg = seg;
  p.scan = (seg != N);
  p.fused = p.scan && fused;
  p.r_split = (p.scan && !p.fused) ? pieces(seg, d, dt, ch) : 1;
  p.nseg = ceil_div(total, seg);
  p.ws_bytes = !p.scan ? 0 : p.fused ? fused_ws_bytes(p.nseg, H, d) : phased_ws_bytes(p, H, d);
  return p;
}

// Packed plan.  Equal cuts of the token axis (seg > 0), with the segment
// scan handing states across cuts; or, for kSegPerSeq, one segment per
// sequence (seg == 0): no hand-off, so no local-state pass, no scan and no
// workspace, and the output pass alone is launched (it also gives empty
// sequences their final state).
Plan plan_varlen(int num_seqs, int H, int64_t total, int d, la_dtype dt,
                 int64_t segment_tokens, bool allow_fused = true, bool ch = false,
                 int block = 128, bool short_ok = false) {
  const int T = out_chunk(d, dt, ch,
                          level_block(block, num_seqs > 0 ? ceil_div(total, num_seqs) : total),
                          short_ok);
  if (segment_tokens == kSegPerSeq) return Plan{0, num_seqs, false, false, 1, 0, T};
  Plan p{1, 0, true, false, 1, 0, T};
  if (total == 0) return p;
  const bool fused = allow_fused && T == la::mfma::T && want_fused(H, d, dt, ch);
  int64_t seg = segment_tokens;
  if (seg <= 0) {
    const int64_t G = ceil_div(target_groups(d, dt, ch, T), H);
    seg = ceil_div(ceil_div(total, G), T) * T;
    if (fused && seg > kFusedSeg) seg = kFusedSeg;
  }
  p.seg = seg;
  p.fused = fused;
  p.r_split = fused ? 1 : pieces(seg, d, dt, ch);
  p.nseg = ceil_div(total, seg);
  p.ws_bytes = fused ? fused_ws_bytes(p.nseg, H, d) : phased_ws_bytes(p, H, d);
  return p;
}

thread_local hipError_t g_last_hip_error = hipSuccess;

la_status launch_status() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) g_last_hip_error = e;
  return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

template <typename Tin, int D, bool CH>
void launch_simt_ch(const la::FwdArgs &a, const Plan &pl, hipStream_t st, bool phase_a) {
  dim3 grid((unsigned)(pl.nseg * a.m.H));
  if (phase_a)
    hipLaunchKernelGGL((la::simt::local_state_kernel<Tin, D, CH>), grid, dim3(la::simt::NT), 0, st,
                       a);
  else
    hipLaunchKernelGGL((la::simt::prefill_chunk_kernel<Tin, D, CH>), grid, dim3(la::simt::NT), 0,
                       st, a);
}

template <typename Tin, int D>
void launch_simt(const la::FwdArgs &a, const Plan &pl, hipStream_t st, bool phase_a) {
  if (a.chdecay)
    launch_simt_ch<Tin, D, true>(a, pl, st, phase_a);
  else
    launch_simt_ch<Tin, D, false>(a, pl, st, phase_a);
}

void launch_phase(const la::FwdArgs &a, const Plan &pl, int d, la_dtype dt, hipStream_t st,
                  bool phase_a) {
  dim3 grid((unsigned)(pl.nseg * a.m.H));
  if (use_mfma(d, dt, a.chdecay != nullptr)) {
    if (phase_a) {
      // The last segment hands no state on: its local state is never needed.
      const dim3 lgrid((unsigned)((pl.nseg - 1) * a.r_split * a.m.H));
      const bool silu_kv = (a.flags & (la::mfma::GF_SILU_K | la::mfma::GF_SILU_V)) != 0;
      if (pl.nseg > 1 && a.chdecay)
        hipLaunchKernelGGL((la::mfma::local_state_kernel<true, false>), lgrid,
                           dim3(la::mfma::NT_LOCAL), 0, st, a);
      else if (pl.nseg > 1 && silu_kv)
        hipLaunchKernelGGL((la::mfma::local_state_kernel<false, true>), lgrid,
                           dim3(la::mfma::NT_LOCAL), 0, st, a);
      else if (pl.nseg > 1)
        hipLaunchKernelGGL((la::mfma::local_state_kernel<false, false>), lgrid,
                           dim3(la::mfma::NT_LOCAL), 0, st, a);
    } else if (pl.chunk < la::mfma::T && !a.chdecay) {
      // Short chunks: two 4-wave workgroups per CU.
      if (pl.chunk == 32)
        hipLaunchKernelGGL((la::mfma::prefill_short_kernel<32>), grid, dim3(la::mfma::NT_S), 0,
                           st, a);
      else
        hipLaunchKernelGGL((la::mfma::prefill_short_kernel<64>), grid, dim3(la::mfma::NT_S), 0,
                           st, a);
    } else if (a.chdecay) {
      // Heads whose smallest decay is at least 1/8 on MFMA, the others on
      // the vector-ALU kernel (same segments, same entering states).
      la::FwdArgs am = a, av = a;
      am.ch_split = 1;
      av.ch_split = 2;
      hipLaunchKernelGGL(la::mfma::chdecay_chunk_kernel, grid, dim3(la::mfma::NT), 0, st, am);
      hipLaunchKernelGGL((la::simt::prefill_chunk_kernel<bf16, 128, true>), grid,
                         dim3(la::simt::NT), 0, st, av);
    } else if (a.flags) {
      // The gated reading's parts compiled in (their own kernels, so that the
      // plain path keeps its registers).
      if (a.seg_len == 0)
        hipLaunchKernelGGL((la::mfma::prefill_chunk_kernel<true, true>), grid, dim3(la::mfma::NT),
                           0, st, a);
      else
        hipLaunchKernelGGL((la::mfma::prefill_chunk_kernel<false, true>), grid, dim3(la::mfma::NT),
                           0, st, a);
    } else if (a.m.snap_iv > 0 || a.seg_len == 0 || a.m.rs < 0) {
      hipLaunchKernelGGL(la::mfma::prefill_chunk_kernel<true>, grid, dim3(la::mfma::NT), 0, st, a);
    } else {
      hipLaunchKernelGGL(la::mfma::prefill_chunk_kernel<false>, grid, dim3(la::mfma::NT), 0, st, a);
    }
  } else if (dt == LA_BF16 && d == 64) {
    launch_simt<bf16, 64>(a, pl, st, phase_a);
  } else if (d == 64) {
    launch_simt<float, 64>(a, pl, st, phase_a);
  } else {
    launch_simt<float, 128>(a, pl, st, phase_a);
  }
}

// Runs the whole prefill for a planned problem (fixed or packed).
// Records phase event i on st when the caller supplied events (a timing
// diagnostic); remembers a failure for the call's status.
struct PhaseEvents {
  void *const *ev;
  hipStream_t st;
  bool failed = false;
  void mark(int i) {
    if (!ev) return;
    const hipError_t e = hipEventRecord((hipEvent_t)ev[i], st);
    if (e != hipSuccess) {
      failed = true;
      g_last_hip_error = e;
    }
  }
};

// out_pass = false: only the local-state pass and the scan (the segment
// entering states), for a caller that launches the output pass itself.
la_status run_fwd(const la::FwdArgs &base, const Plan &pl, int d, la_dtype dt, bool has_empty,
                  hipStream_t st, void *const *events = nullptr, bool out_pass = true) {
  la::FwdArgs a = base;
  const int H = a.m.H;
  a.r_split = pl.r_split;
  // A time-reversed packed view's output pass runs only in the paired
  // backward kernel (the single-pass chunk kernels leave that term out).
  if (a.m.rev_rs != 0 && (pl.fused || (out_pass && use_mfma(d, dt, a.chdecay != nullptr))))
    return LA_ERR_UNSUPPORTED;
  PhaseEvents pe{events, st};
  pe.mark(0);
  if (pl.fused && pl.nseg > 0) {
    // flags, ticket and error word live right after the end-state records
    unsigned *words = (unsigned *)((char *)a.ws + state_bytes(pl.nseg * H, d));
    const int nwords = (int)(pl.nseg * H + 2);
    hipLaunchKernelGGL(la::mfma::fused_reset_kernel, dim3((unsigned)ceil_div(nwords, 256)),
                       dim3(256), 0, st, words, nwords);
    if (has_empty) {
      la::ScanArgs s{a.m, a.decay, pl.seg, 0, d, a.init, a.fin, a.ws, 1, la::mfma::T, nullptr};
      hipLaunchKernelGGL(la::segment_scan_kernel<1>,
                         dim3((unsigned)H, (unsigned)ceil_div((int64_t)d * d, 1024)), dim3(256), 0,
                         st, s);
    }
    pe.mark(1);
    pe.mark(2);
    la::mfma::FusedArgs fa{a, words, words + pl.nseg * H, words + pl.nseg * H + 1};
    if (a.m.snap_iv > 0)
      hipLaunchKernelGGL(la::mfma::prefill_fused_kernel<true>, dim3((unsigned)(pl.nseg * H)),
                         dim3(la::mfma::NT), 0, st, fa);
    else
      hipLaunchKernelGGL(la::mfma::prefill_fused_kernel<false>, dim3((unsigned)(pl.nseg * H)),
                         dim3(la::mfma::NT), 0, st, fa);
    pe.mark(3);
    const la_status ls = launch_status();
    return ls != LA_OK ? ls : pe.failed ? LA_ERR_HIP : LA_OK;
  }
  if (pl.scan && pl.nseg > 0) {
    launch_phase(a, pl, d, dt, st, /*phase_a=*/true);
  }
  pe.mark(1);
  if (pl.scan || has_empty) {
    la::ScanArgs s;
    s.m = a.m;
    s.decay = a.decay;
    s.seg_len = pl.seg;
    s.nseg = pl.scan ? (int)pl.nseg : 0;
    s.d = d;
    s.init = a.init;
    s.fin = a.fin;
    s.ws = a.ws;
    s.r_split = pl.r_split;
    s.C = use_mfma(d, dt, a.chdecay != nullptr) ? la::mfma::C_LOCAL : la::simt::T;
    s.chdecay = a.chdecay;
    s.state_scale = a.state_scale;
    dim3 grid((unsigned)H, (unsigned)ceil_div((int64_t)d * d, 1024));
    switch (pl.r_split) {
      case 16: hipLaunchKernelGGL(la::segment_scan_kernel<16>, grid, dim3(256), 0, st, s); break;
      case 8: hipLaunchKernelGGL(la::segment_scan_kernel<8>, grid, dim3(256), 0, st, s); break;
      case 4: hipLaunchKernelGGL(la::segment_scan_kernel<4>, grid, dim3(256), 0, st, s); break;
      case 2: hipLaunchKernelGGL(la::segment_scan_kernel<2>, grid, dim3(256), 0, st, s); break;
      default: hipLaunchKernelGGL(la::segment_scan_kernel<1>, grid, dim3(256), 0, st, s); break;
    }
  }
  pe.mark(2);
  if (pl.nseg > 0 && out_pass) {
    if (!pl.scan) a.ws = nullptr;
    launch_phase(a, pl, d, dt, st, /*phase_a=*/false);
  }
  pe.mark(3);
  const la_status ls = launch_status();
  return ls != LA_OK ? ls : pe.failed ? LA_ERR_HIP : LA_OK;
}

// Tensors the kernels access with 16-byte vector loads and stores (inputs,
// outputs, states, workspace) must start on a 16-byte boundary; NULL (an
// absent optional tensor) passes.
bool aligned16(std::initializer_list<const void *> ps) {
  for (const void *p : ps)
    if (((uintptr_t)p & 15u) != 0) return false;
  return true;
}

la_status check_common(int H, int d, int block, la_dtype dt, int64_t segment_tokens) {
  if (H < 0 || (segment_tokens < 0 && segment_tokens != kSegPerSeq)) return LA_ERR_INVALID_ARG;
  if (!valid_dtype(dt) || !valid_d(d) || !valid_block(block)) return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

la_status check_layout(la_layout layout, int H, int d) {
  if (layout != LA_HEAD_MAJOR && layout != LA_TOKEN_MAJOR) return LA_ERR_UNSUPPORTED;
  // Output rows are stored through 32-bit byte offsets within a chunk: 128
  // token-major row strides must stay below 2^31 bytes.
  if (layout == LA_TOKEN_MAJOR && (int64_t)H * d * 4 * 128 >= ((int64_t)1 << 31))
    return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

// Kernel arguments of a fixed-length prefill, [B][H][N][d] or [B][N][H][d].
// reversed: a time-reversed view of the same buffers (token t of a sequence
// read and written as token N - 1 - t): the row stride is negated and the
// sequence base moved to the last token, which is still linear in the
// sequence index, so the kernels' addressing is unchanged.
la::FwdArgs fixed_args(const void *q, const void *k, const void *v, void *out, const float *decay,
                       int B, int H, int64_t N, int d, la_dtype dt, la_layout layout,
                       const float *init, float *fin, const Plan &pl, void *workspace,
                       bool reversed) {
  la::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.decay = decay;
  a.m.cu = nullptr;
  a.m.N = N;
  a.m.num_seqs = B;
  a.m.H = H;
  a.m.total = (int64_t)B * N;
  a.m.snap_iv = 0;
  a.m.rev_rs = 0;
  a.snaps = nullptr;
  a.snap_off = nullptr;
  a.chdecay = nullptr;
  if (layout == LA_HEAD_MAJOR) {  // [B][H][N][d]: token t of sequence j, head h at
    a.m.head_stride = N * d;      // ((j H + h) N + t) d = h N d + j (H - 1) N d + (j N + t) d
    a.m.seq_extra = (int64_t)(H - 1) * N * d;
    a.m.rs = d;
  } else {                         // [B][N][H][d]: ((j N + t) H + h) d
    a.m.head_stride = d;
    a.m.seq_extra = 0;
    a.m.rs = (int64_t)H * d;
  }
  if (reversed && N > 0) {
    // Virtual token j N + u is token N - 1 - u of sequence j: element offset
    // base + h hs + j se + (j N + N - 1 - u) rs
    //   = [base + (N - 1) rs] + h hs + j (se + 2 N rs) + (j N + u) (-rs).
    const size_t esz = dt == LA_BF16 ? 2 : 4;
    const int64_t shift = (N - 1) * a.m.rs * (int64_t)esz;
    a.q = (const char *)q + shift;
    a.k = (const char *)k + shift;
    a.v = (const char *)v + shift;
    a.out = (char *)out + shift;
    a.m.seq_extra += 2 * N * a.m.rs;
    a.m.rs = -a.m.rs;
  }
  a.seg_len = pl.seg;
  a.nseg = (int)pl.nseg;
  a.init = init;
  a.fin = fin;
  a.ws = (float *)workspace;
  return a;
}

// The gated path's extras (normalisation, SiLU, gate): none by default.
struct Gated {
  int flags = 0;
  const void *gate = nullptr;
  const float *norm_w = nullptr;
  float eps = 0.f;
  bool entry = false;  // a gated entry point: always the three-phase plan
};

la_status check_gated(const Gated &gt, int d, la_dtype dt) {
  if (gt.flags & ~(LA_SILU_Q | LA_SILU_K | LA_SILU_V | LA_NORM | LA_GATE))
    return LA_ERR_INVALID_ARG;
  if ((gt.flags & LA_GATE) && !gt.gate) return LA_ERR_INVALID_ARG;
  if (!(gt.eps >= 0.f) || !(gt.eps < __builtin_huge_valf())) return LA_ERR_INVALID_ARG;
  if (!aligned16({gt.gate, gt.norm_w})) return LA_ERR_INVALID_ARG;
  if (!(dt == LA_BF16 && d == 128)) return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

void apply_gated(la::FwdArgs &a, const Gated &gt) {
  a.flags = gt.flags;
  a.gate = gt.gate;
  a.norm_w = gt.norm_w;
  a.eps = gt.eps;
}

la_status fwd_fixed(const void *q, const void *k, const void *v, const float *decay, int B, int H,
                    int64_t N, int d, int block, la_dtype dt, la_layout layout,
                    const float *init_state, void *out, float *final_state,
                    int64_t segment_tokens, void *workspace, size_t workspace_bytes,
                    void *hip_stream, void *const *phase_events, const Gated &gt = Gated()) {
  if (B < 0 || N < 0) return LA_ERR_INVALID_ARG;
  la_status st = check_common(H, d, block, dt, segment_tokens);
  if (st == LA_OK) st = check_layout(layout, H, d);
  if (st != LA_OK) return st;
  if ((int64_t)B * H == 0) return LA_OK;
  if (!decay) return LA_ERR_INVALID_ARG;
  if (N > 0 && (!q || !k || !v || !out)) return LA_ERR_INVALID_ARG;
  if (!aligned16({q, k, v, out, init_state, final_state, workspace})) return LA_ERR_INVALID_ARG;
  if ((int64_t)B * N > ((int64_t)1 << 40)) return LA_ERR_UNSUPPORTED;
  const Plan pl = plan_fixed(B, H, N, d, dt, segment_tokens, !gt.entry, false, block, true);
  if (!plan_fits(pl, H)) return LA_ERR_UNSUPPORTED;
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return LA_ERR_WORKSPACE;
  if (N == 0 && !final_state) return LA_OK;

  la::FwdArgs a = fixed_args(q, k, v, out, decay, B, H, N, d, dt, layout, init_state,
                             final_state, pl, workspace, /*reversed=*/false);
  apply_gated(a, gt);
  return run_fwd(a, pl, d, dt, /*has_empty=*/N == 0, (hipStream_t)hip_stream, phase_events);
}

// A validated packed prefill, ready to launch.
struct VarlenCall {
  la::FwdArgs a;
  Plan pl;
  int d;
  la_dtype dt;
  bool launch;  // false: nothing to do
};

la_status prep_varlen(const void *q, const void *k, const void *v, const float *decay,
                      const int32_t *cu_seqlens, int num_seqs, int H, int64_t total_N, int d,
                      int block, la_dtype dt, la_layout layout, const float *init_states,
                      void *out, float *final_states, int64_t segment_tokens, void *workspace,
                      size_t workspace_bytes, int64_t snap_iv, const int32_t *snap_off,
                      float *snaps, VarlenCall *c, bool allow_fused = true,
                      bool ch = false, bool short_ok = false, const Gated &gt = Gated()) {
  c->launch = false;
  if (num_seqs < 0 || total_N < 0 || snap_iv < 0) return LA_ERR_INVALID_ARG;
  if (snap_iv > 0 && snap_iv <= total_N && (!snap_off || !snaps)) return LA_ERR_INVALID_ARG;
  la_status st = check_common(H, d, block, dt, segment_tokens);
  if (st == LA_OK) st = check_layout(layout, H, d);
  if (st != LA_OK) return st;
  if ((int64_t)num_seqs * H == 0) return total_N == 0 ? LA_OK : LA_ERR_INVALID_ARG;
  if (!decay || !cu_seqlens) return LA_ERR_INVALID_ARG;
  if (total_N > 0 && (!q || !k || !v || !out)) return LA_ERR_INVALID_ARG;
  if (!aligned16({q, k, v, out, init_states, final_states, workspace, snaps}))
    return LA_ERR_INVALID_ARG;
  if (total_N > ((int64_t)1 << 40)) return LA_ERR_UNSUPPORTED;
  Plan pl = plan_varlen(num_seqs, H, total_N, d, dt, segment_tokens, allow_fused && !gt.entry,
                        ch, block, short_ok);
  if (!plan_fits(pl, H)) return LA_ERR_UNSUPPORTED;
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return LA_ERR_WORKSPACE;
  // Prefix snapshots are stored by the 128-token kernel; the segments (and
  // so the workspace) stay those of the size query for the same block.
  if (snap_iv > 0 && pl.chunk < la::mfma::T) pl.chunk = la::mfma::T;

  la::FwdArgs &a = c->a;
  a.chdecay = nullptr;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.decay = decay;
  a.m.cu = cu_seqlens;
  a.m.N = 0;
  a.m.num_seqs = num_seqs;
  a.m.H = H;
  a.m.total = total_N;
  a.m.seq_extra = 0;
  a.m.rev_rs = 0;
  // An interval longer than every sequence yields no snapshot.
  a.m.snap_iv = (snap_iv > 0 && snap_iv <= total_N) ? snap_iv : 0;
  a.snaps = a.m.snap_iv ? snaps : nullptr;
  a.snap_off = a.m.snap_iv ? snap_off : nullptr;
  if (layout == LA_HEAD_MAJOR) {  // [H][total_N][d]
    a.m.head_stride = total_N * d;
    a.m.rs = d;
  } else {                         // [total_N][H][d]
    a.m.head_stride = d;
    a.m.rs = (int64_t)H * d;
  }
  a.seg_len = pl.seg;
  a.nseg = (int)pl.nseg;
  a.init = init_states;
  a.fin = final_states;
  a.ws = (float *)workspace;
  apply_gated(a, gt);
  c->pl = pl;
  c->d = d;
  c->dt = dt;
  c->launch = true;
  return LA_OK;
}

// Zero-length sequences get their final state from the scan kernel, except
// with one segment per sequence, where the output pass writes it.
bool varlen_has_empty(const Plan &pl) { return pl.seg != 0; }

la_status fwd_varlen(const void *q, const void *k, const void *v, const float *decay,
                     const int32_t *cu_seqlens, int num_seqs, int H, int64_t total_N, int d,
                     int block, la_dtype dt, la_layout layout, const float *init_states, void *out,
                     float *final_states, int64_t segment_tokens, void *workspace,
                     size_t workspace_bytes, void *hip_stream, int64_t snap_iv = 0,
                     const int32_t *snap_off = nullptr, float *snaps = nullptr,
                     const Gated &gt = Gated()) {
  VarlenCall c;
  const la_status st = prep_varlen(q, k, v, decay, cu_seqlens, num_seqs, H, total_N, d, block, dt,
                                   layout, init_states, out, final_states, segment_tokens,
                                   workspace, workspace_bytes, snap_iv, snap_off, snaps, &c,
                                   /*allow_fused=*/true, /*ch=*/false, /*short_ok=*/true, gt);
  if (st != LA_OK || !c.launch) return st;
  return run_fwd(c.a, c.pl, c.d, c.dt, varlen_has_empty(c.pl), (hipStream_t)hip_stream);
}

// Decode: validation, then the launch.
la_status check_decode(const void *q, const void *k, const void *v, const float *decay,
                       const float *state, const void *out, int B, int H, int d, la_dtype dt) {
  if (B < 0 || H < 0) return LA_ERR_INVALID_ARG;
  if (!valid_dtype(dt) || !valid_d(d)) return LA_ERR_UNSUPPORTED;
  if ((int64_t)B * H == 0) return LA_OK;
  if (!q || !k || !v || !decay || !state || !out) return LA_ERR_INVALID_ARG;
  if (!aligned16({q, k, v, state, out})) return LA_ERR_INVALID_ARG;
  if ((int64_t)B * H > (int64_t)0xffffffff / 256) return LA_ERR_UNSUPPORTED;  // grid x 256
  return LA_OK;
}

template <bool CH>
void launch_decode_t(const void *q, const void *k, const void *v, const float *decay,
                     float *state, void *out, int B, int H, int d, la_dtype dt, hipStream_t st) {
  if ((int64_t)B * H == 0) return;
  dim3 grid((unsigned)((int64_t)B * H));
  if (dt == LA_BF16) {
    if (d == 128)
      hipLaunchKernelGGL((la::decode_kernel<bf16, 128, CH>), grid, dim3(256), 0, st,
                         (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, decay, state,
                         (bf16 *)out, H);
    else
      hipLaunchKernelGGL((la::decode_kernel<bf16, 64, CH>), grid, dim3(256), 0, st,
                         (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, decay, state,
                         (bf16 *)out, H);
  } else {
    if (d == 128)
      hipLaunchKernelGGL((la::decode_kernel<float, 128, CH>), grid, dim3(256), 0, st,
                         (const float *)q, (const float *)k, (const float *)v, decay, state,
                         (float *)out, H);
    else
      hipLaunchKernelGGL((la::decode_kernel<float, 64, CH>), grid, dim3(256), 0, st,
                         (const float *)q, (const float *)k, (const float *)v, decay, state,
                         (float *)out, H);
  }
}

void launch_decode(const void *q, const void *k, const void *v, const float *decay, float *state,
                   void *out, int B, int H, int d, la_dtype dt, hipStream_t st) {
  launch_decode_t<false>(q, k, v, decay, state, out, B, H, d, dt, st);
}

// Channel-wise decay prefill (fixed length): the vector-ALU kernels with
// per-channel decays; the three-phase schedule (never the single-pass one).
la_status fwd_chdecay(const void *q, const void *k, const void *v, const float *alpha, int B,
                      int H, int64_t N, int d, int block, la_dtype dt, la_layout layout,
                      const float *init_state, void *out, float *final_state,
                      int64_t segment_tokens, void *workspace, size_t workspace_bytes,
                      void *hip_stream) {
  if (B < 0 || N < 0) return LA_ERR_INVALID_ARG;
  la_status st = check_common(H, d, block, dt, segment_tokens);
  if (st == LA_OK) st = check_layout(layout, H, d);
  if (st != LA_OK) return st;
  if ((int64_t)B * H == 0) return LA_OK;
  if (!alpha) return LA_ERR_INVALID_ARG;
  if (N > 0 && (!q || !k || !v || !out)) return LA_ERR_INVALID_ARG;
  if (!aligned16({q, k, v, out, init_state, final_state, workspace})) return LA_ERR_INVALID_ARG;
  if ((int64_t)B * N > ((int64_t)1 << 40)) return LA_ERR_UNSUPPORTED;
  const Plan pl = plan_fixed(B, H, N, d, dt, segment_tokens, /*allow_fused=*/false, /*ch=*/true);
  if (!plan_fits(pl, H)) return LA_ERR_UNSUPPORTED;
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return LA_ERR_WORKSPACE;
  if (N == 0 && !final_state) return LA_OK;
  la::FwdArgs a = fixed_args(q, k, v, out, nullptr, B, H, N, d, dt, layout, init_state,
                             final_state, pl, workspace, /*reversed=*/false);
  a.chdecay = alpha;
  return run_fwd(a, pl, d, dt, /*has_empty=*/N == 0, (hipStream_t)hip_stream);
}

// Channel-wise decay over packed sequences: the packed prefill's arguments
// with alpha [H][d] in place of the per-head decay.  One segment per
// sequence is not offered (the channel-wise output pass takes plain
// segments only).
la_status fwd_chdecay_varlen(const void *q, const void *k, const void *v, const float *alpha,
                             const int32_t *cu_seqlens, int num_seqs, int H, int64_t total_N,
                             int d, int block, la_dtype dt, la_layout layout,
                             const float *init_states, void *out, float *final_states,
                             int64_t segment_tokens, void *workspace, size_t workspace_bytes,
                             void *hip_stream) {
  if (segment_tokens == kSegPerSeq) return LA_ERR_UNSUPPORTED;
  VarlenCall c;
  // (alpha is validated where the packed prefill validates the decay)
  const la_status st = prep_varlen(q, k, v, alpha, cu_seqlens, num_seqs, H, total_N, d, block,
                                   dt, layout, init_states, out, final_states, segment_tokens,
                                   workspace, workspace_bytes, 0, nullptr, nullptr, &c,
                                   /*allow_fused=*/false, /*ch=*/true);
  if (st != LA_OK || !c.launch) return st;
  c.a.decay = nullptr;
  c.a.chdecay = alpha;
  return run_fwd(c.a, c.pl, c.d, c.dt, varlen_has_empty(c.pl), (hipStream_t)hip_stream);
}

// The segment entering states a forward keeps for its backward (transposed,
// [nseg][H][d][d]); none when the plan has no scan (every segment starts a
// sequence, from its initial state).
size_t saved_states_bytes(const Plan &pl, int H, int d) {
  return pl.scan ? state_bytes(pl.nseg * H, d) : 0;
}

// Workspace of the backward pass: the passes' prefill workspace (reused by
// all three, which run in stream order), then four state sets of B*H*d*d
// floats (init^T, dS_fin / lambda, its transpose, the dv pass's final
// state), then the dk pass's segment entering states (nseg*H*d*d floats,
// when the plan cuts segments).
size_t bwd_ws_bytes(const Plan &pl, int B, int H, int d) {
  const size_t al = 256;
  return (pl.ws_bytes + al - 1) / al * al + 4 * state_bytes((int64_t)B * H, d) +
         (pl.scan ? state_bytes(pl.nseg * H, d) : 0);
}

// The backward pass on a planned problem.  args(q', k', v', out', init,
// fin, reversed) builds the kernel arguments of one pass over the caller's
// buffers (reversed: the time-reversed view); S = number of state sets
// (batch entries or sequences); has_empty: a scan must also give empty
// sequences their states.
template <typename ArgFn>
la_status bwd_core(const ArgFn &args, const Plan &pl, int S, int H, int d, la_dtype dt,
                   const float *decay, const void *q, const void *k, const void *v,
                   const void *dout, const float *dfinal, const float *init, void *dq, void *dk,
                   void *dv, float *dinit, bool any_token, bool has_empty, void *workspace,
                   hipStream_t s, const float *saved = nullptr) {
  const int64_t SH = (int64_t)S * H;
  const dim3 sgrid((unsigned)SH, (unsigned)ceil_div((int64_t)d * d, 256));
  if (!any_token) {  // no token at all: dS_init = dS_fin
    if (dinit) {
      hipLaunchKernelGGL(la::bwd_dinit_kernel, sgrid, dim3(256), 0, s, dfinal, decay, H, d, false,
                         dinit);
      return launch_status();
    }
    return LA_OK;
  }
  char *w = (char *)workspace;
  const size_t st_b = state_bytes(SH, d);
  float *initT = (float *)(w + (pl.ws_bytes + 255) / 256 * 256);
  float *g = (float *)((char *)initT + st_b);
  float *gT = (float *)((char *)g + st_b);
  float *fin_dv = (float *)((char *)gT + st_b);
  float *dk_in = (float *)((char *)fin_dv + st_b);  // dk pass entering states (pl.scan)
  const dim3 tgrid((unsigned)SH, (unsigned)(d / 32), (unsigned)(d / 32));
  // MFMA path: dv and dk come from one fused pass whose dk side reads the
  // dv pass's state transposed, so the dk pass's own states (gT, dk_in) are
  // not formed.
  const bool fused_dkdv = use_mfma(d, dt);
  if (init)
    hipLaunchKernelGGL(la::transpose_states_kernel, tgrid, dim3(256), 0, s, init, 1, H, d, decay,
                       false, initT);
  // (The fused pass takes dS_fin itself and applies 1 / lambda as it reads
  // it, and lambda as it writes d init: no separate scaling launches.)
  if (dfinal && !fused_dkdv) {
    hipLaunchKernelGGL(la::bwd_scale_kernel, sgrid, dim3(256), 0, s, dfinal, decay, H, d, g);
    hipLaunchKernelGGL(la::transpose_states_kernel, tgrid, dim3(256), 0, s, dfinal, 1, H, d,
                       decay, true, gT);
  }
  // dq: causal, from S_init^T.  Its state is S_t^T, so with the forward's
  // saved segment entering states (transposed) only its output pass runs.
  la_status r;
  if (saved && pl.scan) {
    la::FwdArgs aq = args(dout, v, k, dq, init ? initT : nullptr, nullptr, false);
    aq.ws = const_cast<float *>(saved);
    aq.r_split = 1;
    if (pl.nseg > 0) launch_phase(aq, pl, d, dt, s, /*phase_a=*/false);
    r = launch_status();
  } else {
    r = run_fwd(args(dout, v, k, dq, init ? initT : nullptr, nullptr, false), pl, d, dt,
                has_empty, s);
  }
  // dv: reversed, keys q and values do, from dS_fin / lambda; its final
  // state is G_0.  dk: reversed, keys do and values q, from
  // (dS_fin / lambda)^T.  The dk pass's state is G^T over the same segments,
  // so with segments its entering states are the dv pass's (left in the
  // workspace by the scan) transposed: only the dv pass runs the local-state
  // pass and the scan.
  la::FwdArgs av = fused_dkdv ? args(k, q, dout, dv, dfinal, dinit, true)
                              : args(k, q, dout, dv, dfinal ? g : nullptr, dinit ? fin_dv : nullptr,
                                     true);
  if (fused_dkdv) av.state_scale = 3;
  la::FwdArgs ak = args(v, dout, q, dk, dfinal ? gT : nullptr, nullptr, true);
  if (r == LA_OK) r = run_fwd(av, pl, d, dt, has_empty, s, nullptr, /*out_pass=*/false);
  if (r == LA_OK) {
    if (pl.scan) {
      if (!fused_dkdv)
        hipLaunchKernelGGL(la::transpose_states_kernel,
                           dim3((unsigned)(pl.nseg * H), (unsigned)(d / 32), (unsigned)(d / 32)),
                           dim3(256), 0, s, (const float *)workspace, pl.r_split, H, d, decay,
                           false, dk_in);
      av.r_split = pl.r_split;
      ak.ws = dk_in;
      ak.r_split = 1;
    } else {
      av.ws = nullptr;
      ak.ws = nullptr;
    }
    if (pl.nseg > 0) {
      if (fused_dkdv) {
        // Both output passes in one workgroup per (segment, head).
        if (av.m.rev_rs != 0)
          hipLaunchKernelGGL(la::mfma::prefill_dkdv_kernel<true>, dim3((unsigned)(pl.nseg * H)),
                             dim3(la::mfma::NT), 0, s, av, ak);
        else
          hipLaunchKernelGGL(la::mfma::prefill_dkdv_kernel<false>, dim3((unsigned)(pl.nseg * H)),
                             dim3(la::mfma::NT), 0, s, av, ak);
      } else {
        launch_phase(av, pl, d, dt, s, /*phase_a=*/false);
        launch_phase(ak, pl, d, dt, s, /*phase_a=*/false);
      }
    }
    r = launch_status();
  }
  if (r == LA_OK && dinit && !fused_dkdv) {
    hipLaunchKernelGGL(la::bwd_dinit_kernel, sgrid, dim3(256), 0, s, fin_dv, decay, H, d, true,
                       dinit);
    r = launch_status();
  }
  return r;
}

la_status bwd_fixed(const void *q, const void *k, const void *v, const float *decay,
                    const void *dout, const float *dfinal, const float *init, void *dq, void *dk,
                    void *dv, float *dinit, int B, int H, int64_t N, int d, int block,
                    la_dtype dt, la_layout layout, int64_t segment_tokens, void *workspace,
                    size_t workspace_bytes, void *hip_stream, bool with_saved = false,
                    const float *saved = nullptr, size_t saved_bytes = 0) {
  if (B < 0 || N < 0) return LA_ERR_INVALID_ARG;
  la_status st = check_common(H, d, block, dt, segment_tokens);
  if (st == LA_OK) st = check_layout(layout, H, d);
  if (st != LA_OK) return st;
  if ((int64_t)B * H == 0) return LA_OK;
  if (!decay) return LA_ERR_INVALID_ARG;
  if (N > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv)) return LA_ERR_INVALID_ARG;
  if (!aligned16({q, k, v, dout, dq, dk, dv, dfinal, init, dinit, workspace, saved}))
    return LA_ERR_INVALID_ARG;
  if ((int64_t)B * N > ((int64_t)1 << 40)) return LA_ERR_UNSUPPORTED;
  const Plan pl = plan_fixed(B, H, N, d, dt, segment_tokens, /*allow_fused=*/false);
  if (!plan_fits(pl, H)) return LA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < bwd_ws_bytes(pl, B, H, d)) return LA_ERR_WORKSPACE;
  if (with_saved && saved_bytes < saved_states_bytes(pl, H, d)) return LA_ERR_INVALID_ARG;
  if (with_saved && saved_states_bytes(pl, H, d) > 0 && !saved) return LA_ERR_INVALID_ARG;
  auto args = [&](const void *q_, const void *k_, const void *v_, void *o_, const float *init_,
                  float *fin_, bool reversed) {
    return fixed_args(q_, k_, v_, o_, decay, B, H, N, d, dt, layout, init_, fin_, pl, workspace,
                      reversed);
  };
  return bwd_core(args, pl, B, H, d, dt, decay, q, k, v, dout, dfinal, init, dq, dk, dv, dinit,
                  N > 0, /*has_empty=*/false, workspace, (hipStream_t)hip_stream,
                  with_saved ? saved : nullptr);
}

la_status bwd_varlen(const void *q, const void *k, const void *v, const float *decay,
                     const void *dout, const int32_t *cu_seqlens, int num_seqs, int H,
                     int64_t total_N, int d, int block, la_dtype dt, la_layout layout,
                     const float *dfinals, const float *inits, void *dq, void *dk, void *dv,
                     float *dinits, int64_t segment_tokens, void *workspace,
                     size_t workspace_bytes, void *hip_stream, bool with_saved = false,
                     const float *saved = nullptr, size_t saved_bytes = 0) {
  if (num_seqs < 0 || total_N < 0) return LA_ERR_INVALID_ARG;
  la_status st = check_common(H, d, block, dt, segment_tokens);
  if (st == LA_OK) st = check_layout(layout, H, d);
  if (st != LA_OK) return st;
  if ((int64_t)num_seqs * H == 0) return total_N == 0 ? LA_OK : LA_ERR_INVALID_ARG;
  if (!decay || !cu_seqlens) return LA_ERR_INVALID_ARG;
  if (total_N > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv)) return LA_ERR_INVALID_ARG;
  if (!aligned16({q, k, v, dout, dq, dk, dv, dfinals, inits, dinits, workspace, saved}))
    return LA_ERR_INVALID_ARG;
  if (total_N > ((int64_t)1 << 40)) return LA_ERR_UNSUPPORTED;
  const Plan pl = plan_varlen(num_seqs, H, total_N, d, dt, segment_tokens, /*allow_fused=*/false);
  if (!plan_fits(pl, H)) return LA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < bwd_ws_bytes(pl, num_seqs, H, d)) return LA_ERR_WORKSPACE;
  if (with_saved && saved_bytes < saved_states_bytes(pl, H, d)) return LA_ERR_INVALID_ARG;
  if (with_saved && saved_states_bytes(pl, H, d) > 0 && !saved) return LA_ERR_INVALID_ARG;
  la::FwdArgs base;
  base.decay = decay;
  base.chdecay = nullptr;
  base.snaps = nullptr;
  base.snap_off = nullptr;
  base.r_split = 1;
  base.m.cu = cu_seqlens;
  base.m.N = 0;
  base.m.num_seqs = num_seqs;
  base.m.H = H;
  base.m.total = total_N;
  base.m.seq_extra = 0;
  base.m.snap_iv = 0;
  base.m.rev_rs = 0;
  if (layout == LA_HEAD_MAJOR) {  // [H][total_N][d]
    base.m.head_stride = total_N * d;
    base.m.rs = d;
  } else {                         // [total_N][H][d]
    base.m.head_stride = d;
    base.m.rs = (int64_t)H * d;
  }
  auto args = [&](const void *q_, const void *k_, const void *v_, void *o_, const float *init_,
                  float *fin_, bool reversed) {
    la::FwdArgs a = base;
    a.q = q_;
    a.k = k_;
    a.v = v_;
    a.out = o_;
    a.init = init_;
    a.fin = fin_;
    a.seg_len = pl.seg;
    a.nseg = (int)pl.nseg;
    a.ws = (float *)workspace;
    if (reversed) {  // token u of sequence j read as token start(j+1) - 1 - u
      a.m.rev_rs = a.m.rs;
      a.m.rs = -a.m.rs;
    }
    return a;
  };
  return bwd_core(args, pl, num_seqs, H, d, dt, decay, q, k, v, dout, dfinals, inits, dq, dk, dv,
                  dinits, total_N > 0, varlen_has_empty(pl), workspace,
                  (hipStream_t)hip_stream, with_saved ? saved : nullptr);
}

// The forward of a training pair: the three-phase schedule of the backward's
// plan, then the scan's segment entering states, transposed, into saved.
la_status fwd_save(const void *q, const void *k, const void *v, const float *decay, int B, int H,
                   int64_t N, int d, int block, la_dtype dt, la_layout layout,
                   const float *init_state, void *out, float *final_state,
                   int64_t segment_tokens, float *saved, size_t saved_bytes, void *workspace,
                   size_t workspace_bytes, void *hip_stream) {
  if (B < 0 || N < 0) return LA_ERR_INVALID_ARG;
  la_status st = check_common(H, d, block, dt, segment_tokens);
  if (st == LA_OK) st = check_layout(layout, H, d);
  if (st != LA_OK) return st;
  if ((int64_t)B * H == 0) return LA_OK;
  if (!decay) return LA_ERR_INVALID_ARG;
  if (N > 0 && (!q || !k || !v || !out)) return LA_ERR_INVALID_ARG;
  if (!aligned16({q, k, v, out, init_state, final_state, workspace})) return LA_ERR_INVALID_ARG;
  if ((int64_t)B * N > ((int64_t)1 << 40)) return LA_ERR_UNSUPPORTED;
  const Plan pl = plan_fixed(B, H, N, d, dt, segment_tokens, /*allow_fused=*/false);
  if (!plan_fits(pl, H)) return LA_ERR_UNSUPPORTED;
  const size_t need = saved_states_bytes(pl, H, d);
  if (saved_bytes < need || (need > 0 && !saved) || !aligned16({saved}))
    return LA_ERR_INVALID_ARG;
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return LA_ERR_WORKSPACE;
  if (N == 0 && !final_state) return LA_OK;
  const la::FwdArgs a = fixed_args(q, k, v, out, decay, B, H, N, d, dt, layout, init_state,
                                   final_state, pl, workspace, /*reversed=*/false);
  const hipStream_t s = (hipStream_t)hip_stream;
  la_status r = run_fwd(a, pl, d, dt, /*has_empty=*/N == 0, s);
  if (r == LA_OK && need > 0) {
    hipLaunchKernelGGL(la::transpose_states_kernel,
                       dim3((unsigned)(pl.nseg * H), (unsigned)(d / 32), (unsigned)(d / 32)),
                       dim3(256), 0, s, (const float *)workspace, pl.r_split, H, d, decay, false,
                       saved);
    r = launch_status();
  }
  return r;
}

// The packed forward of a training pair (as fwd_save).
la_status fwd_varlen_save(const void *q, const void *k, const void *v, const float *decay,
                          const int32_t *cu_seqlens, int num_seqs, int H, int64_t total_N, int d,
                          int block, la_dtype dt, la_layout layout, const float *init_states,
                          void *out, float *final_states, int64_t segment_tokens, float *saved,
                          size_t saved_bytes, void *workspace, size_t workspace_bytes,
                          void *hip_stream) {
  VarlenCall c;
  la_status st = prep_varlen(q, k, v, decay, cu_seqlens, num_seqs, H, total_N, d, block, dt,
                             layout, init_states, out, final_states, segment_tokens, workspace,
                             workspace_bytes, 0, nullptr, nullptr, &c, /*allow_fused=*/false);
  if (st != LA_OK || !c.launch) return st;
  const size_t need = saved_states_bytes(c.pl, H, d);
  if (saved_bytes < need || (need > 0 && !saved) || !aligned16({saved}))
    return LA_ERR_INVALID_ARG;
  const hipStream_t s = (hipStream_t)hip_stream;
  st = run_fwd(c.a, c.pl, d, dt, varlen_has_empty(c.pl), s);
  if (st == LA_OK && need > 0) {
    hipLaunchKernelGGL(la::transpose_states_kernel,
                       dim3((unsigned)(c.pl.nseg * H), (unsigned)(d / 32), (unsigned)(d / 32)),
                       dim3(256), 0, s, (const float *)workspace, c.pl.r_split, H, d, decay,
                       false, saved);
    st = launch_status();
  }
  return st;
}

// Scratch of lightning_attn_fwd_noalloc: the workspace of a prefill, held in
// the library instead of coming from the caller (256 MiB: the partial states
// of the local-state pass at the 1M-token 8-head shape, 32 segments x 16
// pieces x 8 heads x 64 KiB; 64 MiB at the 64-head 32768-token shape).  Every GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address comes
// from hipGetSymbolAddress, once per device (scratch_address below).
constexpr size_t kScratchBytes = (size_t)256 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up on the
// first call on that device (with that device current) and kept.
la_status scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = e;
    return LA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return LA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      g_last_hip_error = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return LA_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LA_OK;
}

}  // namespace

extern "C" {

size_t lightning_attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

la_status lightning_attn_fwd_noalloc(const void *q, const void *k, const void *v,
                                     const float *decay, int B, int H, int64_t N, int d,
                                     int block, la_dtype dt, const float *init_state, void *out,
                                     float *final_state, int64_t segment_tokens,
                                     void *hip_stream) {
  void *ws = nullptr;
  const la_status st = scratch_address(&ws);
  if (st != LA_OK) return st;
  return fwd_fixed(q, k, v, decay, B, H, N, d, block, dt, LA_HEAD_MAJOR, init_state, out,
                   final_state, segment_tokens, ws, kScratchBytes, hip_stream, nullptr);
}

size_t lightning_attn_fwd_chdecay_varlen_workspace_size(int num_seqs, int H, int64_t total_N,
                                                        int d, int block, la_dtype dt,
                                                        int64_t segment_tokens) {
  if (num_seqs < 0 || total_N < 0 || check_common(H, d, block, dt, segment_tokens) != LA_OK)
    return 0;
  if ((int64_t)num_seqs * H == 0 || segment_tokens == kSegPerSeq) return 0;
  return plan_varlen(num_seqs, H, total_N, d, dt, segment_tokens, false, true).ws_bytes;
}

la_status lightning_attn_fwd_chdecay_varlen(const void *q, const void *k, const void *v,
                                            const float *alpha, const int32_t *cu_seqlens,
                                            int num_seqs, int H, int64_t total_N, int d,
                                            int block, la_dtype dt, la_layout layout,
                                            const float *init_states, void *out,
                                            float *final_states, int64_t segment_tokens,
                                            void *workspace, size_t workspace_bytes,
                                            void *hip_stream) {
  return fwd_chdecay_varlen(q, k, v, alpha, cu_seqlens, num_seqs, H, total_N, d, block, dt,
                            layout, init_states, out, final_states, segment_tokens, workspace,
                            workspace_bytes, hip_stream);
}

size_t lightning_attn_fwd_chdecay_workspace_size(int B, int H, int64_t N, int d, int block,
                                                 la_dtype dt, int64_t segment_tokens) {
  if (B < 0 || N < 0 || check_common(H, d, block, dt, segment_tokens) != LA_OK) return 0;
  if ((int64_t)B * H == 0) return 0;
  return plan_fixed(B, H, N, d, dt, segment_tokens, false, true).ws_bytes;
}

la_status lightning_attn_fwd_chdecay(const void *q, const void *k, const void *v,
                                     const float *alpha, int B, int H, int64_t N, int d, int block,
                                     la_dtype dt, la_layout layout, const float *init_state,
                                     void *out, float *final_state, int64_t segment_tokens,
                                     void *workspace, size_t workspace_bytes, void *hip_stream) {
  return fwd_chdecay(q, k, v, alpha, B, H, N, d, block, dt, layout, init_state, out, final_state,
                     segment_tokens, workspace, workspace_bytes, hip_stream);
}

size_t lightning_attn_saved_states_size(int B, int H, int64_t N, int d, int block, la_dtype dt,
                                        int64_t segment_tokens) {
  if (B < 0 || N < 0 || check_common(H, d, block, dt, segment_tokens) != LA_OK) return 0;
  if ((int64_t)B * H == 0) return 0;
  return saved_states_bytes(plan_fixed(B, H, N, d, dt, segment_tokens, false), H, d);
}

la_status lightning_attn_fwd_save(const void *q, const void *k, const void *v, const float *decay,
                                  int B, int H, int64_t N, int d, int block, la_dtype dt,
                                  la_layout layout, const float *init_state, void *out,
                                  float *final_state, int64_t segment_tokens, float *saved,
                                  size_t saved_bytes, void *workspace, size_t workspace_bytes,
                                  void *hip_stream) {
  return fwd_save(q, k, v, decay, B, H, N, d, block, dt, layout, init_state, out, final_state,
                  segment_tokens, saved, saved_bytes, workspace, workspace_bytes, hip_stream);
}

la_status lightning_attn_bwd_saved(const void *q, const void *k, const void *v, const float *decay,
                                   const void *dout, const float *dfinal, const float *init_state,
                                   void *dq, void *dk, void *dv, float *dinit, int B, int H,
                                   int64_t N, int d, int block, la_dtype dt, la_layout layout,
                                   int64_t segment_tokens, const float *saved, size_t saved_bytes,
                                   void *workspace, size_t workspace_bytes, void *hip_stream) {
  return bwd_fixed(q, k, v, decay, dout, dfinal, init_state, dq, dk, dv, dinit, B, H, N, d, block,
                   dt, layout, segment_tokens, workspace, workspace_bytes, hip_stream,
                   /*with_saved=*/true, saved, saved_bytes);
}

size_t lightning_attn_varlen_saved_states_size(int num_seqs, int H, int64_t total_N, int d,
                                               int block, la_dtype dt, int64_t segment_tokens) {
  if (num_seqs < 0 || total_N < 0 || check_common(H, d, block, dt, segment_tokens) != LA_OK)
    return 0;
  if ((int64_t)num_seqs * H == 0) return 0;
  return saved_states_bytes(plan_varlen(num_seqs, H, total_N, d, dt, segment_tokens, false), H,
                            d);
}

la_status lightning_attn_fwd_varlen_save(const void *q, const void *k, const void *v,
                                         const float *decay, const int32_t *cu_seqlens,
                                         int num_seqs, int H, int64_t total_N, int d, int block,
                                         la_dtype dt, la_layout layout, const float *init_states,
                                         void *out, float *final_states, int64_t segment_tokens,
                                         float *saved, size_t saved_bytes, void *workspace,
                                         size_t workspace_bytes, void *hip_stream) {
  return fwd_varlen_save(q, k, v, decay, cu_seqlens, num_seqs, H, total_N, d, block, dt, layout,
                         init_states, out, final_states, segment_tokens, saved, saved_bytes,
                         workspace, workspace_bytes, hip_stream);
}

la_status lightning_attn_bwd_varlen_saved(const void *q, const void *k, const void *v,
                                          const float *decay, const void *dout,
                                          const int32_t *cu_seqlens, int num_seqs, int H,
                                          int64_t total_N, int d, int block, la_dtype dt,
                                          la_layout layout, const float *dfinals,
                                          const float *init_states, void *dq, void *dk, void *dv,
                                          float *dinits, int64_t segment_tokens,
                                          const float *saved, size_t saved_bytes,
                                          void *workspace, size_t workspace_bytes,
                                          void *hip_stream) {
  return bwd_varlen(q, k, v, decay, dout, cu_seqlens, num_seqs, H, total_N, d, block, dt, layout,
                    dfinals, init_states, dq, dk, dv, dinits, segment_tokens, workspace,
                    workspace_bytes, hip_stream, /*with_saved=*/true, saved, saved_bytes);
}

size_t lightning_attn_bwd_workspace_size(int B, int H, int64_t N, int d, int block, la_dtype dt,
                                         int64_t segment_tokens) {
  if (B < 0 || N < 0 || check_common(H, d, block, dt, segment_tokens) != LA_OK) return 0;
  if ((int64_t)B * H == 0) return 0;
  return bwd_ws_bytes(plan_fixed(B, H, N, d, dt, segment_tokens, false), B, H, d);
}

size_t lightning_attn_bwd_varlen_workspace_size(int num_seqs, int H, int64_t total_N, int d,
                                                int block, la_dtype dt, int64_t segment_tokens) {
  if (num_seqs < 0 || total_N < 0 || check_common(H, d, block, dt, segment_tokens) != LA_OK)
    return 0;
  if ((int64_t)num_seqs * H == 0) return 0;
  return bwd_ws_bytes(plan_varlen(num_seqs, H, total_N, d, dt, segment_tokens, false), num_seqs,
                      H, d);
}

la_status lightning_attn_bwd_varlen(const void *q, const void *k, const void *v,
                                    const float *decay, const void *dout,
                                    const int32_t *cu_seqlens, int num_seqs, int H,
                                    int64_t total_N, int d, int block, la_dtype dt,
                                    la_layout layout, const float *dfinals,
                                    const float *init_states, void *dq, void *dk, void *dv,
                                    float *dinits, int64_t segment_tokens, void *workspace,
                                    size_t workspace_bytes, void *hip_stream) {
  return bwd_varlen(q, k, v, decay, dout, cu_seqlens, num_seqs, H, total_N, d, block, dt, layout,
                    dfinals, init_states, dq, dk, dv, dinits, segment_tokens, workspace,
                    workspace_bytes, hip_stream);
}

la_status lightning_attn_bwd(const void *q, const void *k, const void *v, const float *decay,
                             const void *dout, const float *dfinal, const float *init_state,
                             void *dq, void *dk, void *dv, float *dinit, int B, int H, int64_t N,
                             int d, int block, la_dtype dt, la_layout layout,
                             int64_t segment_tokens, void *workspace, size_t workspace_bytes,
                             void *hip_stream) {
  return bwd_fixed(q, k, v, decay, dout, dfinal, init_state, dq, dk, dv, dinit, B, H, N, d, block,
                   dt, layout, segment_tokens, workspace, workspace_bytes, hip_stream);
}


const char *lightning_attn_status_string(la_status s) {
  switch (s) {
    case LA_OK: return "ok";
    case LA_ERR_INVALID_ARG: return "invalid argument";
    case LA_ERR_UNSUPPORTED: return "unsupported configuration";
    case LA_ERR_WORKSPACE: return "workspace missing or too small";
    case LA_ERR_HIP: return "HIP launch error";
    default: break;
  }
  return "unknown status";
}

int lightning_attn_version(void) { return kVersion; }

const char *lightning_attn_last_hip_error(void) {
  return g_last_hip_error == hipSuccess ? "no HIP error" : hipGetErrorString(g_last_hip_error);
}

size_t lightning_attn_fwd_workspace_size(int B, int H, int64_t N, int d, int block, la_dtype dt,
                                         int64_t segment_tokens) {
  if (B < 0 || N < 0 || check_common(H, d, block, dt, segment_tokens) != LA_OK) return 0;
  if ((int64_t)B * H == 0) return 0;
  return plan_fixed(B, H, N, d, dt, segment_tokens, true, false, block, true).ws_bytes;
}

la_status lightning_attn_fwd(const void *q, const void *k, const void *v, const float *decay,
                             int B, int H, int64_t N, int d, int block, la_dtype dt,
                             const float *init_state, void *out, float *final_state,
                             int64_t segment_tokens, void *workspace, size_t workspace_bytes,
                             void *hip_stream) {
  return fwd_fixed(q, k, v, decay, B, H, N, d, block, dt, LA_HEAD_MAJOR, init_state, out,
                   final_state, segment_tokens, workspace, workspace_bytes, hip_stream, nullptr);
}

la_status lightning_attn_fwd_timed(const void *q, const void *k, const void *v,
                                   const float *decay, int B, int H, int64_t N, int d, int block,
                                   la_dtype dt, const float *init_state, void *out,
                                   float *final_state, int64_t segment_tokens, void *workspace,
                                   size_t workspace_bytes, void *hip_stream,
                                   void *const *phase_events) {
  return fwd_fixed(q, k, v, decay, B, H, N, d, block, dt, LA_HEAD_MAJOR, init_state, out,
                   final_state, segment_tokens, workspace, workspace_bytes, hip_stream,
                   phase_events);
}

la_status lightning_attn_fwd_layout(const void *q, const void *k, const void *v,
                                    const float *decay, int B, int H, int64_t N, int d, int block,
                                    la_dtype dt, la_layout layout, const float *init_state,
                                    void *out, float *final_state, int64_t segment_tokens,
                                    void *workspace, size_t workspace_bytes, void *hip_stream) {
  return fwd_fixed(q, k, v, decay, B, H, N, d, block, dt, layout, init_state, out, final_state,
                   segment_tokens, workspace, workspace_bytes, hip_stream, nullptr);
}

size_t lightning_attn_fwd_varlen_workspace_size(int num_seqs, int H, int64_t total_N, int d,
                                                int block, la_dtype dt, int64_t segment_tokens) {
  if (num_seqs < 0 || total_N < 0 || check_common(H, d, block, dt, segment_tokens) != LA_OK)
    return 0;
  if ((int64_t)num_seqs * H == 0) return 0;
  return plan_varlen(num_seqs, H, total_N, d, dt, segment_tokens, true, false, block, true)
      .ws_bytes;
}

la_status lightning_attn_fwd_varlen(const void *q, const void *k, const void *v,
                                    const float *decay, const int32_t *cu_seqlens, int num_seqs,
                                    int H, int64_t total_N, int d, int block, la_dtype dt,
                                    const float *init_states, void *out, float *final_states,
                                    int64_t segment_tokens, void *workspace,
                                    size_t workspace_bytes, void *hip_stream) {
  return fwd_varlen(q, k, v, decay, cu_seqlens, num_seqs, H, total_N, d, block, dt, LA_HEAD_MAJOR,
                    init_states, out, final_states, segment_tokens, workspace, workspace_bytes,
                    hip_stream);
}

la_status lightning_attn_fwd_varlen_layout(const void *q, const void *k, const void *v,
                                           const float *decay, const int32_t *cu_seqlens,
                                           int num_seqs, int H, int64_t total_N, int d, int block,
                                           la_dtype dt, la_layout layout,
                                           const float *init_states, void *out,
                                           float *final_states, int64_t segment_tokens,
                                           void *workspace, size_t workspace_bytes,
                                           void *hip_stream) {
  return fwd_varlen(q, k, v, decay, cu_seqlens, num_seqs, H, total_N, d, block, dt, layout,
                    init_states, out, final_states, segment_tokens, workspace, workspace_bytes,
                    hip_stream);
}

la_status lightning_attn_fwd_varlen_snapshots(
    const void *q, const void *k, const void *v, const float *decay, const int32_t *cu_seqlens,
    int num_seqs, int H, int64_t total_N, int d, int block, la_dtype dt, la_layout layout,
    const float *init_states, void *out, float *final_states, int64_t snapshot_interval,
    const int32_t *snapshot_offsets, float *snapshots, int64_t segment_tokens, void *workspace,
    size_t workspace_bytes, void *hip_stream) {
  if (snapshot_interval < 1) return LA_ERR_INVALID_ARG;
  return fwd_varlen(q, k, v, decay, cu_seqlens, num_seqs, H, total_N, d, block, dt, layout,
                    init_states, out, final_states, segment_tokens, workspace, workspace_bytes,
                    hip_stream, snapshot_interval, snapshot_offsets, snapshots);
}

la_status lightning_attn_decode(const void *q, const void *k, const void *v, const float *decay,
                                float *state, void *out, int B, int H, int d, la_dtype dt,
                                void *hip_stream) {
  const la_status st = check_decode(q, k, v, decay, state, out, B, H, d, dt);
  if (st != LA_OK) return st;
  if ((int64_t)B * H == 0) return LA_OK;
  launch_decode(q, k, v, decay, state, out, B, H, d, dt, (hipStream_t)hip_stream);
  return launch_status();
}

la_status lightning_attn_decode_chdecay(const void *q, const void *k, const void *v,
                                        const float *alpha, float *state, void *out, int B, int H,
                                        int d, la_dtype dt, void *hip_stream) {
  const la_status st = check_decode(q, k, v, alpha, state, out, B, H, d, dt);
  if (st != LA_OK) return st;
  if ((int64_t)B * H == 0) return LA_OK;
  launch_decode_t<true>(q, k, v, alpha, state, out, B, H, d, dt, (hipStream_t)hip_stream);
  return launch_status();
}

la_status lightning_attn_mixed_step(
    const void *prefill_q, const void *prefill_k, const void *prefill_v,
    const int32_t *cu_seqlens, int num_seqs, int64_t total_N, la_layout layout,
    const float *init_states, void *prefill_out, float *final_states, int64_t segment_tokens,
    void *workspace, size_t workspace_bytes, void *prefill_stream, const void *decode_q,
    const void *decode_k, const void *decode_v, float *decode_state, void *decode_out,
    int decode_B, void *decode_stream, const float *decay, int H, int d, int block,
    la_dtype dt) {
  // Both parts are validated before either launches.
  VarlenCall c;
  la_status st = prep_varlen(prefill_q, prefill_k, prefill_v, decay, cu_seqlens, num_seqs, H,
                             total_N, d, block, dt, layout, init_states, prefill_out,
                             final_states, segment_tokens, workspace, workspace_bytes, 0,
                             nullptr, nullptr, &c, /*allow_fused=*/true, /*ch=*/false,
                             /*short_ok=*/true);
  if (st != LA_OK) return st;
  st = check_decode(decode_q, decode_k, decode_v, decay, decode_state, decode_out, decode_B, H, d,
                    dt);
  if (st != LA_OK) return st;
  // The prefill chain (up to three launches) goes first so that it starts
  // at once; the decode kernel's many small workgroups fill the CUs the
  // prefill leaves free.
  la_status sp = LA_OK;
  if (c.launch)
    sp = run_fwd(c.a, c.pl, c.d, c.dt, varlen_has_empty(c.pl), (hipStream_t)prefill_stream);
  la_status sd = LA_OK;
  if ((int64_t)decode_B * H > 0) {
    launch_decode(decode_q, decode_k, decode_v, decay, decode_state, decode_out, decode_B, H, d,
                  dt, (hipStream_t)decode_stream);
    sd = launch_status();
  }
  return sp != LA_OK ? sp : sd;
}

// The gated entry points run the 128-token kernel (the normalisation and
// gate compiled into it) in the three-phase schedule.
constexpr int kGatedBlock = 128;

size_t lightning_attn_fwd_gated_workspace_size(int B, int H, int64_t N, int d, la_dtype dt,
                                               int64_t segment_tokens) {
  if (B < 0 || N < 0 || check_common(H, d, kGatedBlock, dt, segment_tokens) != LA_OK) return 0;
  if ((int64_t)B * H == 0) return 0;
  return plan_fixed(B, H, N, d, dt, segment_tokens, false, false, kGatedBlock, true).ws_bytes;
}

la_status lightning_attn_fwd_gated(const void *q, const void *k, const void *v,
                                   const float *decay, int B, int H, int64_t N, int d,
                                   la_dtype dt, la_layout layout, int flags, const void *gate,
                                   const float *norm_weight, float eps,
                                   const float *init_state, void *out, float *final_state,
                                   int64_t segment_tokens, void *workspace,
                                   size_t workspace_bytes, void *hip_stream) {
  Gated gt;
  gt.flags = flags;
  gt.gate = gate;
  gt.norm_w = norm_weight;
  gt.eps = eps;
  gt.entry = true;
  if (B < 0 || N < 0 || H < 0) return LA_ERR_INVALID_ARG;
  const la_status st = check_gated(gt, d, dt);
  if (st != LA_OK) return st;
  return fwd_fixed(q, k, v, decay, B, H, N, d, kGatedBlock, dt, layout, init_state, out,
                   final_state, segment_tokens, workspace, workspace_bytes, hip_stream, nullptr,
                   gt);
}

size_t lightning_attn_fwd_varlen_gated_workspace_size(int num_seqs, int H, int64_t total_N, int d,
                                                      la_dtype dt, int64_t segment_tokens) {
  if (num_seqs < 0 || total_N < 0 ||
      check_common(H, d, kGatedBlock, dt, segment_tokens) != LA_OK)
    return 0;
  if ((int64_t)num_seqs * H == 0) return 0;
  return plan_varlen(num_seqs, H, total_N, d, dt, segment_tokens, false, false, kGatedBlock, true)
      .ws_bytes;
}

la_status lightning_attn_fwd_varlen_gated(const void *q, const void *k, const void *v,
                                          const float *decay, const int32_t *cu_seqlens,
                                          int num_seqs, int H, int64_t total_N, int d,
                                          la_dtype dt, la_layout layout, int flags,
                                          const void *gate, const float *norm_weight, float eps,
                                          const float *init_states, void *out,
                                          float *final_states, int64_t segment_tokens,
                                          void *workspace, size_t workspace_bytes,
                                          void *hip_stream) {
  Gated gt;
  gt.flags = flags;
  gt.gate = gate;
  gt.norm_w = norm_weight;
  gt.eps = eps;
  gt.entry = true;
  if (num_seqs < 0 || total_N < 0 || H < 0) return LA_ERR_INVALID_ARG;
  const la_status st = check_gated(gt, d, dt);
  if (st != LA_OK) return st;
  return fwd_varlen(q, k, v, decay, cu_seqlens, num_seqs, H, total_N, d, kGatedBlock, dt, layout,
                    init_states, out, final_states, segment_tokens, workspace, workspace_bytes,
                    hip_stream, 0, nullptr, nullptr, gt);
}

}  // extern "C"

#ifdef LA_PHASE_PROBE
// The phase-timing build's extra entry points (not in the public header:
// the library proper is built without them).
extern "C" int lightning_attn_phase_probe_copy(void *dst, size_t bytes) {
  if (bytes > sizeof(la::mfma::g_phase_probe)) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(la::mfma::g_phase_probe), bytes, 0,
                                  hipMemcpyDeviceToHost);
}
extern "C" int lightning_attn_phase_probe_copy_local(void *dst, size_t bytes) {
  if (bytes > sizeof(la::mfma::g_phase_probe_local)) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(la::mfma::g_phase_probe_local), bytes, 0,
                                  hipMemcpyDeviceToHost);
}
extern "C" int lightning_attn_phase_probe_clear(void) {
  void *a = nullptr, *b = nullptr;
  hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(la::mfma::g_phase_probe));
  if (e == hipSuccess) e = hipGetSymbolAddress(&b, HIP_SYMBOL(la::mfma::g_phase_probe_local));
  if (e == hipSuccess) e = hipMemset(a, 0, sizeof(la::mfma::g_phase_probe));
  if (e == hipSuccess) e = hipMemset(b, 0, sizeof(la::mfma::g_phase_probe_local));
  return (int)e;
}
#endif
