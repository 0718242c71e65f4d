// Segment scan (phase B) and the decode step.
#pragma once

#include "la_common.h"

namespace la {

// Phase B, the on-device analogue of LASP+ (MiniMax-01 report, section
// 3.2.2 and Fig. 12(b)): every segment's local state L_s is known; the state
// entering segment s is
//   S_in[s] = init(j)                         if a sequence j starts at a_s
//           = gamma_{s-1} base_{s-1} + L_{s-1}  otherwise,
// with gamma = lambda^(length of the segment's last piece) and base the state
// entering that piece (S_in of the segment, or init of the piece's sequence
// when that sequence starts inside the segment).  ws holds the partial local
// states of each segment's pieces on entry (L_s is their decayed sum) and
// S_in[s] at the segment's first slot on exit.  Also writes final states of
// zero-length sequences.
// Grid: (H, d*d / 1024), items spread over the XCDs (xcd_spread); each
// thread owns 4 consecutive state elements.
struct ScanArgs {
  SeqMap m;
  const float *decay;
  int64_t seg_len;
  int nseg;
  int d;
  const float *init;
  float *fin;
  float *ws;     // [nseg][r_split][H][d][d]: partial local states in, S_in at slot (s, 0) out
  int r_split;   // pieces per segment of the local-state pass: 1, 2, 4, 8 or 16
  int C;         // chunk length of the local-state pass
  const float *chdecay;  // [H][d] per-channel decays, or nullptr (scalar decay)
  int state_scale;       // as FwdArgs::state_scale (0 unless set)
};

// What the scan needs of segment s, computed once per workgroup.
struct SegInfo {
  int init_in;    // sequence whose initial state enters the segment, or -1 (carry)
  int init_base;  // sequence whose initial state is the last piece's base, or -1
                  // (the base is the entering state)
  int hands_on;   // the segment's last sequence continues after it
  int live;       // bit r: piece r of the local-state pass was computed
  float gam;      // lambda^(length of the last piece)
  float wt[16];   // lambda^(b - x1_r): weight of piece r in L_s
  float gam_n;    // the exponents of gam and wt (channel-wise decay: each
  float wt_n[16]; // state row raises its own decay to them)
};

__device__ __forceinline__ SegInfo describe(const ScanArgs &p, const SeqMap &m, int s,
                                            float log2lam) {
  SegInfo d;
  const int64_t a = (int64_t)s * p.seg_len;
  const int64_t b = (a + p.seg_len < m.total) ? a + p.seg_len : m.total;
  const int jf = m.seq_of(a);
  d.init_in = (m.start(jf) == a) ? jf : -1;
  const int jl = m.seq_of(b - 1);
  const int64_t ps0 = m.start(jl);
  const int64_t ps = ps0 > a ? ps0 : a;
  d.init_base = (ps == a) ? -1 : jl;
  d.hands_on = m.start(jl + 1) != b;
  d.gam = pow_lam(log2lam, (float)(b - ps));
  d.gam_n = (float)(b - ps);
  // Pieces as the local-state pass cut them (piece_plan); a piece was
  // computed when it is not empty and the state is handed on.
  const Pieces P = piece_plan(ps, b, log2lam, p.C, p.r_split);
  d.live = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    int64_t x0 = b, x1 = b;
    if (r < (1 << P.lg)) piece_range(P, b, p.C, r, &x0, &x1);
    const bool live = d.hands_on && x0 < x1;
    d.live |= live ? (1 << r) : 0;
    d.wt[r] = live ? pow_lam(log2lam, (float)(b - x1)) : 0.f;
    d.wt_n[r] = (float)(b - x1);
  }
  return d;
}

// R = p.r_split, a template parameter so that the partial states of a block
// of segments load into a register array of fixed size.
template <int R>
__global__ __launch_bounds__(256) void segment_scan_kernel(ScanArgs p) {
  constexpr int MAXS = 256;              // segments described per pass
  constexpr int BLK = R >= 16 ? 1 : R >= 8 ? 2 : 4;  // segments loaded together
  __shared__ SegInfo info[MAXS];
  const SeqMap &m = p.m;
  // Items (head, element block), heads fastest, spread over the XCDs (a
  // slowly decaying head has more live pieces to read).
  const int item = xcd_spread((int)(blockIdx.y * gridDim.x + blockIdx.x),
                              (int)(gridDim.x * gridDim.y));
  const int H = m.H, h = item % H;
  const int64_t DD = (int64_t)p.d * p.d;
  const int64_t e = ((int64_t)(item / H) * 256 + threadIdx.x) * 4;
  const bool mine = e < DD;
  // Channel-wise decay: segments are described with the slowest channel's
  // decay (a piece is live if any channel weighs it), and this thread's
  // state row (elements e..e+3 share row e / d) raises its own decay to the
  // described exponents.
  float log2lam, l2row = 0.f;
  if (p.chdecay) {
    const float *al = p.chdecay + (int64_t)h * p.d;
    log2lam = -__builtin_huge_valf();
    for (int i = 0; i < p.d; ++i) log2lam = fmaxf(log2lam, log2f(al[i]));
    l2row = log2f(al[mine ? (int)(e / p.d) : 0]);
  } else {
    log2lam = log2f(p.decay[h]);
  }
  // state_scale bit 0: initial states enter as init / lambda_h.
  const float init_f = (p.state_scale & 1) ? 1.f / p.decay[h] : 1.f;
  auto init4 = [&](int j) -> f32x4 {
    if (!p.init || j < 0) return (f32x4){0.f, 0.f, 0.f, 0.f};
    return init_f * *(const f32x4 *)(p.init + ((int64_t)j * H + h) * DD + e);
  };
  f32x4 carry = {0.f, 0.f, 0.f, 0.f};
  for (int sb = 0; sb < p.nseg; sb += MAXS) {
    const int cnt = (p.nseg - sb) < MAXS ? (p.nseg - sb) : MAXS;
    __syncthreads();
    if ((int)threadIdx.x < cnt) info[threadIdx.x] = describe(p, m, sb + threadIdx.x, log2lam);
    __syncthreads();
    if (!mine) continue;
    for (int s0 = 0; s0 < cnt; s0 += BLK) {
      // Every partial-state load of the block goes out before the
      // (sequential, register-only) carry chain runs through it.
      f32x4 pr[BLK][R];
#pragma unroll
      for (int i = 0; i < BLK; ++i)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const bool live = s0 + i < cnt && ((info[s0 + i].live >> r) & 1);
          pr[i][r] = live ? *(const f32x4 *)(p.ws +
                                             (((int64_t)(sb + s0 + i) * R + r) * H + h) * DD + e)
                          : (f32x4){0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int i = 0; i < BLK; ++i) {
        if (s0 + i >= cnt) break;
        const SegInfo &d = info[s0 + i];
        const f32x4 sin = d.init_in >= 0 ? init4(d.init_in) : carry;
        *(f32x4 *)(p.ws + ((int64_t)(sb + s0 + i) * R * H + h) * DD + e) = sin;
        float wt[R], gam = d.gam;
#pragma unroll
        for (int r = 0; r < R; ++r) wt[r] = d.wt[r];
        if (p.chdecay) {
          gam = pow_lam(l2row, d.gam_n);
#pragma unroll
          for (int r = 0; r < R; ++r)
            wt[r] = ((d.live >> r) & 1) ? pow_lam(l2row, d.wt_n[r]) : 0.f;
        }
        f32x4 loc = wt[0] * pr[i][0];
#pragma unroll
        for (int r = 1; r < R; ++r) loc += wt[r] * pr[i][r];
        const f32x4 base = d.init_base >= 0 ? init4(d.init_base) : sin;
        // When the segment's last sequence ends at b, the carry is unused:
        // the next segment starts a new sequence.
        carry = d.hands_on ? gam * base + loc : (f32x4){0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  if (p.fin && mine) {
    // (bit 1: final states leave as lambda_h times the state)
    const float fin_f = (p.state_scale & 2) ? p.decay[h] : 1.f;
    for (int j = 0; j < m.num_seqs; ++j)
      if (m.start(j) == m.start(j + 1))
        *(f32x4 *)(p.fin + ((int64_t)j * H + h) * DD + e) = fin_f * init4(j);
  }
}

// One decode step for one (sequence, head) per workgroup (MiniMax-01
// report, section 2.2.4, eq. 12; section 3.3.1, fused decode update):
//   S <- lambda S + k^T v;  o = q S.
// The state is streamed once: thread (rg, cg) owns columns 4cg..4cg+3 of
// D/RG consecutive rows; all its loads are issued before any store, and the
// per-row-group partial outputs are summed through LDS.  State loads and
// stores are non-temporal: each byte is touched once per step and a batch's
// state (512 MiB at 128 x 64 heads) is larger than the 256 MB Infinity Cache,
// so keeping it out of the caches frees them for everything else.
// CH: channel-wise decay, decay is [H][D] and row i of the state decays by
// decay[h][i] (S <- diag(alpha) S + k^T v).
template <typename Tin, int D, bool CH = false>
__global__ __launch_bounds__(256) void decode_kernel(const Tin *__restrict__ q,
                                                     const Tin *__restrict__ k,
                                                     const Tin *__restrict__ v,
                                                     const float *__restrict__ decay,
                                                     float *__restrict__ state, Tin *__restrict__ out,
                                                     int H) {
  constexpr int CG = D / 4, RG = 256 / CG, RPT = D / RG;
  __shared__ float qs[D], ks[D], as[CH ? D : 1];
  __shared__ float red[RG][D];
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
  const int64_t bh = blockIdx.x;
  const int h = (int)(bh % H);
  const float lam = CH ? 1.f : decay[h];
  if (tid < D) {
    qs[tid] = to_f32(q[bh * D + tid]);
    ks[tid] = to_f32(k[bh * D + tid]);
    if constexpr (CH) as[tid] = decay[(int64_t)h * D + tid];
  }
  f32x4 vv;
#pragma unroll
  for (int u = 0; u < 4; ++u) vv[u] = to_f32(v[bh * D + 4 * cg + u]);
  f32x4 *S = (f32x4 *)(state + bh * (int64_t)D * D);
  f32x4 sv[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) sv[r] = __builtin_nontemporal_load(&S[(rg * RPT + r) * CG + cg]);
  __syncthreads();
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int i = rg * RPT + r;
    sv[r] = (CH ? as[i] : lam) * sv[r] + ks[i] * vv;
    o += qs[i] * sv[r];
    __builtin_nontemporal_store(sv[r], &S[i * CG + cg]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) red[rg][4 * cg + u] = o[u];
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) acc += red[r][tid];
    out[bh * D + tid] = from_f32<Tin>(acc);
  }
}

}  // namespace la
