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
// when that sequence starts inside the segment).  ws holds L_s on entry and
// S_in[s] on exit.  Also writes final states of zero-length sequences.
// Grid: (H, d*d / 1024); each thread owns 4 consecutive state elements.
struct ScanArgs {
  SeqMap m;
  const float *decay;
  int64_t seg_len;
  int nseg;
  int d;
  const float *init;
  float *fin;
  float *ws;
};

__global__ __launch_bounds__(256) void segment_scan_kernel(ScanArgs p) {
  const SeqMap &m = p.m;
  const int H = m.H, h = blockIdx.x;
  const int64_t DD = (int64_t)p.d * p.d;
  const int64_t e = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4;
  if (e >= DD) return;
  const float log2lam = log2f(p.decay[h]);
  auto init4 = [&](int j) -> f32x4 {
    if (!p.init) return (f32x4){0.f, 0.f, 0.f, 0.f};
    return *(const f32x4 *)(p.init + ((int64_t)j * H + h) * DD + e);
  };
  f32x4 carry = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.nseg; ++s) {
    const int64_t a = (int64_t)s * p.seg_len;
    const int64_t b = (a + p.seg_len < m.total) ? a + p.seg_len : m.total;
    const int jf = m.seq_of(a);
    const f32x4 sin = (m.start(jf) == a) ? init4(jf) : carry;
    f32x4 *slot = (f32x4 *)(p.ws + ((int64_t)s * H + h) * DD + e);
    const f32x4 loc = *slot;
    *slot = sin;
    const int jl = m.seq_of(b - 1);
    const int64_t ps0 = m.start(jl);
    const int64_t ps = ps0 > a ? ps0 : a;
    const float gam = pow_lam(log2lam, (float)(b - ps));
    const f32x4 base = (ps == a) ? sin : init4(jl);
    // When the segment's last sequence ends at b, loc was never written and
    // the carry is unused: the next segment starts a new sequence.
    carry = (m.start(jl + 1) == b) ? (f32x4){0.f, 0.f, 0.f, 0.f} : gam * base + loc;
  }
  if (p.fin) {
    for (int j = 0; j < m.num_seqs; ++j)
      if (m.start(j) == m.start(j + 1))
        *(f32x4 *)(p.fin + ((int64_t)j * H + h) * DD + e) = init4(j);
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
template <typename Tin, int D>
__global__ __launch_bounds__(256) void decode_kernel(const Tin *__restrict__ q,
                                                     const Tin *__restrict__ k,
                                                     const Tin *__restrict__ v,
                                                     const float *__restrict__ decay,
                                                     float *__restrict__ state, Tin *__restrict__ out,
                                                     int H) {
  constexpr int CG = D / 4, RG = 256 / CG, RPT = D / RG;
  __shared__ float qs[D], ks[D];
  __shared__ float red[RG][D];
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
  const int64_t bh = blockIdx.x;
  const int h = (int)(bh % H);
  const float lam = decay[h];
  if (tid < D) {
    qs[tid] = to_f32(q[bh * D + tid]);
    ks[tid] = to_f32(k[bh * D + tid]);
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
    sv[r] = lam * sv[r] + ks[i] * vv;
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
