// Shared device-side definitions for the lightning attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 raw bytes in four registers (a native vector, so register arrays of it
// stay in registers where copies of HIP's struct-based uint4 can be lowered
// to memory copies).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define LA_LDS __attribute__((address_space(3)))

// 2^x on the hardware exponential unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A value that is the same in every lane, moved to a scalar register.
__device__ __forceinline__ float uniform(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// lambda^n for a non-negative integer n, as 2^(n log2 lambda); 0 when the
// power underflows float32 (those terms are below float32 resolution).
__device__ __forceinline__ float pow_lam(float log2lam, float n) { return fast_exp2(n * log2lam); }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Where every sequence lives.  Tokens of one head are numbered in the
// concatenation of all sequences ("virtual" token index); sequence j holds
// virtual tokens start(j) .. start(j+1)-1.  Row g of head h in sequence j is
// at element offset row_base(h, j) + g * d of q, k, v and out.
//   fixed length [B][H][N][d]: start(j) = j N, head_stride = N d,
//                              seq_extra = (H - 1) N d.
//   packed [H][total][d]     : start(j) = cu[j], head_stride = total d,
//                              seq_extra = 0.
// A time-reversed packed view (virtual token start(j) + u is token
// start(j+1) - 1 - u) negates rs and adds (start(j) + start(j+1) - 1) times
// the forward row stride (rev_rs) to row_base.
struct SeqMap {
  const int32_t *cu;  // device cu_seqlens, or nullptr for uniform length N
  int64_t N;
  int num_seqs;
  int H;
  int64_t total;  // tokens per head
  int64_t head_stride;
  int64_t seq_extra;
  int64_t rs;  // elements between consecutive tokens of one head: d (head-major
               // layouts) or H*d (token-major layouts)
  int64_t snap_iv;  // prefix-state snapshot interval in tokens, 0 = none
  int64_t rev_rs;   // time-reversed packed view (0: none): the row stride of the
                    // forward layout; sequence j's base moves to its last token

  __device__ __forceinline__ int64_t start(int j) const {
    return cu ? (int64_t)cu[j] : (int64_t)j * N;
  }
  // The sequence holding virtual token tok (0 <= tok < total): the largest j
  // with start(j) <= tok, which skips zero-length sequences.
  __device__ __forceinline__ int seq_of(int64_t tok) const {
    if (!cu) return (int)(tok / N);
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if ((int64_t)cu[mid] <= tok) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  }
  // REV = false: the caller never sees a time-reversed packed view (rev_rs
  // is 0) and keeps the plain address arithmetic.
  template <bool REV = true>
  __device__ __forceinline__ int64_t row_base(int h, int j) const {
    int64_t r = (int64_t)h * head_stride + (int64_t)j * seq_extra;
    if (REV && rev_rs) r += (start(j) + start(j + 1) - 1) * rev_rs;
    return r;
  }
};

// A chunk [c0, c1) of at most T tokens inside segment [a, b), within the
// piece of sequence j that the segment holds.  Chunks restart at every
// sequence start and stop at every sequence end, at the segment end and at
// every snapshot point (a multiple of snap_iv tokens into the sequence), so
// that the state after a snapshot point's last token exists at a chunk end.
struct Cursor {
  int64_t c0, c1;
  int64_t pend;     // end of the current piece: min(b, seq_end)
  int64_t seq_start;  // start(j)
  int64_t seq_end;  // start(j + 1)
  int64_t snap;     // first snapshot point of sequence j after c0 (INT64_MAX: none)
  int j;
  bool valid;
};

constexpr int64_t kNoSnap = INT64_MAX;

__device__ __forceinline__ int64_t min3(int64_t x, int64_t y, int64_t z) {
  const int64_t t = x < y ? x : y;
  return t < z ? t : z;
}

// SNAP = false compiles the snapshot cuts out (m.snap_iv is ignored), so
// kernels without snapshots keep their scalar registers.
template <bool SNAP>
__device__ __forceinline__ Cursor first_chunk(const SeqMap &m, int64_t a, int64_t b, int T) {
  Cursor c;
  c.valid = a < b;
  c.j = c.valid ? m.seq_of(a) : 0;
  c.seq_start = c.valid ? m.start(c.j) : a;
  c.seq_end = c.valid ? m.start(c.j + 1) : b;
  c.pend = c.seq_end < b ? c.seq_end : b;
  c.snap = kNoSnap;
  if (SNAP && m.snap_iv > 0 && c.valid)
    c.snap = c.seq_start + ((a - c.seq_start) / m.snap_iv + 1) * m.snap_iv;
  c.c0 = a;
  c.c1 = SNAP ? min3(a + T, c.pend, c.snap) : (a + T < c.pend ? a + T : c.pend);
  return c;
}

template <bool SNAP>
__device__ __forceinline__ Cursor next_chunk(const SeqMap &m, const Cursor &c, int64_t b, int T) {
  Cursor n = c;
  n.c0 = c.c1;
  if (n.c0 >= b) {
    n.valid = false;
    return n;
  }
  if (n.c0 >= c.pend) {  // the piece ended at a sequence end: next sequence
    n.j = m.seq_of(n.c0);
    n.seq_start = n.c0;  // start(n.j): seq_of skips empty sequences
    n.seq_end = m.start(n.j + 1);
    n.pend = n.seq_end < b ? n.seq_end : b;
    if (SNAP) n.snap = m.snap_iv > 0 ? n.c0 + m.snap_iv : kNoSnap;  // start(n.j) == n.c0
  } else if (SNAP && n.c0 == c.snap) {
    n.snap = c.snap + m.snap_iv;
  }
  n.c1 = SNAP ? min3(n.c0 + T, n.pend, n.snap) : (n.c0 + T < n.pend ? n.c0 + T : n.pend);
  n.valid = true;
  return n;
}

// SeqMap::row_base(h, c.j) from the bounds the cursor already holds: no
// load of the sequence table (in a chunk loop such a scalar load's wait
// would also wait for every LDS access in flight).
template <bool REV>
__device__ __forceinline__ int64_t chunk_row_base(const SeqMap &m, int h, const Cursor &c) {
  int64_t r = (int64_t)h * m.head_stride + (int64_t)c.j * m.seq_extra;
  if (REV && m.rev_rs) r += (c.seq_start + c.seq_end - 1) * m.rev_rs;
  return r;
}

// Row of `snaps` that receives the state after chunk c (which ends at the
// snapshot point c.snap of sequence c.j): snapshot number
// (c.snap - start(j)) / snap_iv, counted from 1, of that sequence.
__device__ __forceinline__ int64_t snap_row(const SeqMap &m, const int32_t *snap_off,
                                            const Cursor &c) {
  const unsigned n = (unsigned)(c.snap - m.start(c.j)) / (unsigned)m.snap_iv;
  return (int64_t)snap_off[c.j] + (int64_t)n - 1;
}

// First chunk of a local-state pass over [ps, b) (chunks of T tokens
// aligned to ps) that can carry a nonzero weight.  A token more than
// 160 / |log2 lambda| before b has weight lambda^(b-1-c) < 2^-160; every
// float32 step that forms such a weight (2^x of an exponent below -150, and
// its products) yields exactly zero, so whole chunks of such tokens add
// exactly nothing and are skipped: the result is bit-identical.  For
// fast-decaying heads this leaves a few chunks of a segment; lambda = 1 skips
// nothing.
__device__ __forceinline__ int64_t first_weighted(int64_t ps, int64_t b, float log2lam, int T) {
  if (!(log2lam < 0.f)) return ps;  // lambda = 1: every token keeps weight 1
  const float far = (float)(b - ps) + 160.f / log2lam;  // (b - ps) - 160 / |log2 lambda|
  return far >= (float)T ? ps + (int64_t)(far / (float)T) * T : ps;
}

// XCD-aware work order.  MI355X dispatches workgroup i of a launch to XCD
// i mod 8 (8 XCDs of 32 CUs, each with its own L2 and its own share of the
// memory bandwidth).  A grid whose items are ordered heads fastest thus puts
// every item of head h on XCD h mod 8: with 8 heads, a slowly decaying
// head's whole local-state pass (its long pieces) on one XCD.  Kernels whose
// items carry unequal work take item xcd_spread(i, n) in workgroup i
// instead: inside each group of 8 consecutive workgroups the items are
// rotated by the group's index, so items 8 apart (the same head) land on
// different XCDs.  A bijection of [0, n) (the last, partial group keeps its
// order).
__device__ __forceinline__ int xcd_spread(int i, int n) {
  const int j = i >> 3, x = i & 7;
  if ((j + 1) * 8 > n) return i;
  return (j << 3) | ((x + j) & 7);
}

// Arguments shared by the prefill kernels.
struct FwdArgs {
  const void *q, *k, *v;
  void *out;
  const float *decay;
  SeqMap m;
  int64_t seg_len;   // segment length in tokens; 0: segment s is sequence s
  int nseg;          // segments per head
  const float *init; // [S][H][d][d] or nullptr
  float *fin;        // [S][H][d][d] or nullptr
  float *ws;         // segment states (scan mode) or nullptr: [nseg][r_split][H][d][d];
                     // the state entering segment s is at slot (s, 0)
  int r_split;       // pieces per segment of the local-state pass (>= 1)
  float *snaps;      // prefix-state snapshots [rows][H][d][d] (m.snap_iv > 0), else nullptr
  const int32_t *snap_off;  // [num_seqs + 1]: first snapshot row of each sequence
  const float *chdecay;     // [H][d] per-channel decays (channel-wise variant), else nullptr
  int ch_split = 0;         // channel-wise output pass: 0 = every head, 1 = only the heads
                            // whose smallest decay is >= 2^kChMinLog2, 2 = only the others
  int flags = 0;            // gated path: SiLU on q / k / v, normalisation, gate (GF_*)
  const void *gate = nullptr;      // gate input, laid out like out (GF_GATE)
  const float *norm_w = nullptr;   // [H][d] normalisation weight, or nullptr (ones)
  float eps = 0.f;                 // normalisation epsilon
  int state_scale = 0;  // backward's dv pass (fused dv/dk kernel and scan): bit 0, an initial
                        // state is read as init / lambda_h; bit 1, a final state is written
                        // as lambda_h times the state
};

// The channel-wise MFMA output pass writes the decay inside a 64-token
// chunk as alpha^(q-32) (queries) times alpha^(32-c) (keys): factors up to
// alpha^-32, which must stay inside the bf16 range (2^128) with room for the
// inputs themselves.  Heads whose smallest decay is below 2^kChMinLog2 (the
// factors would pass 2^96) run their output pass on the vector-ALU kernel,
// which tabulates the powers and has no such limit.
constexpr float kChMinLog2 = -3.0f;

// True when the smallest of head h's D channel decays is below
// 2^kChMinLog2 (the same value in every lane of the workgroup).
__device__ __forceinline__ bool ch_small_head(const float *alpha_h, int D) {
  float mn = 1.f;
  for (int i = 0; i < D; ++i) mn = fminf(mn, alpha_h[i]);
  return log2f(mn) < kChMinLog2;
}

// Tokens [*a, *b) of segment s: equal cuts of the token axis, or sequence s
// itself when seg_len is 0 (then no segment starts inside a sequence).
__device__ __forceinline__ void segment_bounds(const FwdArgs &p, int s, int64_t *a, int64_t *b) {
  if (p.seg_len == 0) {
    *a = p.m.start(s);
    *b = p.m.start(s + 1);
  } else {
    *a = (int64_t)s * p.seg_len;
    *b = (*a + p.seg_len < p.m.total) ? *a + p.seg_len : p.m.total;
  }
}

// The pieces of a local-state range [ps, b), chunks of C tokens aligned to
// ps: its weighted part [tf, b) (tf = first_weighted) is cut into 2^lg
// pieces of whole chunks, one workgroup each.  A range weighted throughout
// gets R pieces (the plan's piece count, a power of two); one whose leading
// chunks carry zero weight (a faster decay) gets proportionally fewer, so
// that every piece is about as long as a piece of a fully weighted range.
struct Pieces {
  int64_t tf;  // first weighted token (a chunk boundary)
  int64_t nw;  // weighted chunks
  int lg;      // log2 of the piece count
};

__device__ __forceinline__ Pieces piece_plan(int64_t ps, int64_t b, float log2lam, int C, int R) {
  Pieces P;
  P.tf = first_weighted(ps, b, log2lam, C);
  const int64_t n = (b - ps + C - 1) / C;
  P.nw = (b - P.tf + C - 1) / C;
  const int64_t want = n > 0 ? (P.nw * R + n - 1) / n : 1;
  int lg = 0;
  while ((1 << lg) < want && (1 << lg) < R) ++lg;
  P.lg = lg;
  return P;
}

// Piece r (< 2^P.lg) of that cut: chunks [r nw / 2^lg, (r + 1) nw / 2^lg) of
// the weighted part, as tokens [*x0, *x1) (x1 capped at b).  A piece may be
// empty (x0 == x1) when the weighted part has fewer chunks than pieces.
__device__ __forceinline__ void piece_range(const Pieces &P, int64_t b, int C, int r, int64_t *x0,
                                            int64_t *x1) {
  *x0 = P.tf + (((int64_t)r * P.nw) >> P.lg) * C;
  const int64_t e = P.tf + ((((int64_t)r + 1) * P.nw) >> P.lg) * C;
  *x1 = e < b ? e : b;
}

}  // namespace la
