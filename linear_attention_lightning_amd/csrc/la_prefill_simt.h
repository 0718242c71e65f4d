// Vector-ALU prefill for float32 inputs (and bf16 inputs with d = 64):
// the same blockwise schedule as the MFMA path, in float32 throughout, with
// 32-token chunks and the d x d state held in LDS.
//   P = (Q K^T) (.) D,   O = diag(a) Q S + P V,   S = lambda^L S + (diag(b) K)^T V
// (MiniMax-01 report, section 2.2.1: left product inside a block, right
// product between blocks.)
#pragma once

#include "la_common.h"

namespace la {
namespace simt {

constexpr int T = 32;    // tokens per chunk
constexpr int NT = 256;  // threads per workgroup

template <int D>
struct Smem {
  float Q[T][D];
  float K[T][D];
  float V[T][D];
  float S[D][D];
  float P[T][T + 1];
  float bw[T];
};

// Extra LDS of the channel-wise variant: pw[n][i] = alpha_i^n for n < T.
template <int D>
struct SmemCh {
  float pw[T][D];
};

template <typename Tin, int D>
__device__ __forceinline__ void load_rows(float (*dst)[D], const Tin *src, int64_t rs, int L, int tid) {
  for (int e = tid; e < T * D; e += NT) {
    int r = e / D, c = e - (e / D) * D;
    dst[r][c] = r < L ? to_f32(src[(int64_t)r * rs + c]) : 0.f;
  }
}

// CH: channel-wise decay (one decay alpha_i per key channel i, p.chdecay):
//   P[r][c] = sum_i Q[r][i] K[c][i] alpha_i^(r-c),
//   O = (Q (.) alpha^(r+1)) S + P V,
//   S = diag(alpha^L) S + (K (.) alpha^(L-1-c))^T V,
// with the powers alpha_i^n (n < T) tabulated once per workgroup.
template <typename Tin, int D, bool CH = false>
__global__ __launch_bounds__(NT) void prefill_chunk_kernel(FwdArgs p) {
  __shared__ Smem<D> sm;
  __shared__ SmemCh<CH ? D : 1> sc;
  const int tid = threadIdx.x;
  const SeqMap &m = p.m;
  const int H = m.H;
  const int s = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const float log2lam = CH ? 0.f : log2f(p.decay[h]);
  if constexpr (CH) {
    // Beside the MFMA output pass: only the heads it leaves out.
    if (p.ch_split == 2 && !ch_small_head(p.chdecay + (int64_t)h * D, D)) return;
    for (int e = tid; e < T * D; e += NT) {
      const int n = e / D, i = e - (e / D) * D;
      sc.pw[n][i] = pow_lam(log2f(p.chdecay[(int64_t)h * D + i]), (float)n);
    }
  }
  int64_t a, b;
  segment_bounds(p, s, &a, &b);
  const int64_t DD = (int64_t)D * D;
  Cursor cur = first_chunk<true>(m, a, b, T);
  if (!cur.valid) {
    // One segment per sequence: an empty sequence keeps its initial state.
    if (p.seg_len == 0 && p.fin) {
      float *dst = p.fin + ((int64_t)s * H + h) * DD;
      const float *src = p.init ? p.init + ((int64_t)s * H + h) * DD : nullptr;
      for (int e = tid; e < D * D; e += NT) dst[e] = src ? src[e] : 0.f;
    }
    return;
  }
  {
    const float *s0 = p.ws ? p.ws + ((int64_t)s * p.r_split * H + h) * DD
                           : (p.init ? p.init + ((int64_t)cur.j * H + h) * DD : nullptr);
    for (int e = tid; e < D * D; e += NT) (&sm.S[0][0])[e] = s0 ? s0[e] : 0.f;
  }
  constexpr int RSTEP = NT / D;  // output rows handled per pass
  while (true) {
    const int L = (int)(cur.c1 - cur.c0);
    const int64_t base = m.row_base(h, cur.j) + cur.c0 * m.rs;
    load_rows<Tin, D>(sm.Q, (const Tin *)p.q + base, m.rs, L, tid);
    load_rows<Tin, D>(sm.K, (const Tin *)p.k + base, m.rs, L, tid);
    load_rows<Tin, D>(sm.V, (const Tin *)p.v + base, m.rs, L, tid);
    if (tid < T) sm.bw[tid] = tid < L ? pow_lam(log2lam, (float)(L - 1 - tid)) : 0.f;
    __syncthreads();
    // masked, decayed scores
    for (int e = tid; e < T * T; e += NT) {
      int r = e / T, c = e - (e / T) * T;
      float acc = 0.f;
      if (c <= r && r < L) {
        if constexpr (CH) {
          for (int i = 0; i < D; ++i) acc += sm.Q[r][i] * sm.K[c][i] * sc.pw[r - c][i];
        } else {
          for (int i = 0; i < D; ++i) acc += sm.Q[r][i] * sm.K[c][i];
          acc *= pow_lam(log2lam, (float)(r - c));
        }
      }
      sm.P[r][c] = acc;
    }
    __syncthreads();
    // outputs
    {
      const int j = tid % D;
      Tin *obase = (Tin *)p.out + base;
      for (int r = tid / D; r < L; r += RSTEP) {
        float inter = 0.f;
        if constexpr (CH) {
          // alpha_i^(r+1) = alpha_i^r alpha_i^1
          for (int i = 0; i < D; ++i) inter += sm.Q[r][i] * (sc.pw[r][i] * sc.pw[1][i]) * sm.S[i][j];
        } else {
          for (int i = 0; i < D; ++i) inter += sm.Q[r][i] * sm.S[i][j];
          inter *= pow_lam(log2lam, (float)(r + 1));
        }
        float intra = 0.f;
        for (int c = 0; c <= r; ++c) intra += sm.P[r][c] * sm.V[c][j];
        obase[(int64_t)r * m.rs + j] = from_f32<Tin>(inter + intra);
      }
    }
    __syncthreads();
    const Cursor nxt = next_chunk<true>(m, cur, b, T);
    const bool seq_done = (cur.c1 == cur.seq_end);
    const bool new_piece = nxt.valid && (nxt.c0 >= cur.pend);
    const bool snap_here = (cur.c1 == cur.snap);
    if ((nxt.valid && !new_piece) || (seq_done && p.fin) || snap_here) {
      const float gL = pow_lam(log2lam, (float)L);
      for (int e = tid; e < D * D; e += NT) {
        int i = e / D, j = e - (e / D) * D;
        float acc = 0.f;
        if constexpr (CH) {
          // alpha_i^(L-1-c), and alpha_i^L = alpha_i^(L-1) alpha_i
          for (int c = 0; c < L; ++c) acc += (sc.pw[L - 1 - c][i] * sm.K[c][i]) * sm.V[c][j];
          sm.S[i][j] = (sc.pw[L - 1][i] * sc.pw[1][i]) * sm.S[i][j] + acc;
        } else {
          for (int c = 0; c < L; ++c) acc += (sm.bw[c] * sm.K[c][i]) * sm.V[c][j];
          sm.S[i][j] = gL * sm.S[i][j] + acc;
        }
      }
      __syncthreads();
      if (seq_done && p.fin) {
        float *dst = p.fin + ((int64_t)cur.j * H + h) * DD;
        for (int e = tid; e < D * D; e += NT) dst[e] = (&sm.S[0][0])[e];
      }
      if (snap_here) {
        float *dst = p.snaps + (snap_row(m, p.snap_off, cur) * H + h) * DD;
        for (int e = tid; e < D * D; e += NT) dst[e] = (&sm.S[0][0])[e];
      }
    }
    if (!nxt.valid) break;
    __syncthreads();
    if (new_piece) {
      const float *s0 = p.init ? p.init + ((int64_t)nxt.j * H + h) * DD : nullptr;
      for (int e = tid; e < D * D; e += NT) (&sm.S[0][0])[e] = s0 ? s0[e] : 0.f;
    }
    cur = nxt;
  }
}

// Local state of each segment's last piece, from zero (phase A).
// CH: channel-wise decay; token c weighs alpha_i^(b-1-c) in channel i, and
// the zero-weight skip uses the slowest channel's decay.
template <typename Tin, int D, bool CH = false>
__global__ __launch_bounds__(NT) void local_state_kernel(FwdArgs p) {
  __shared__ float Ks[T][D];
  __shared__ float Vs[T][D];
  __shared__ float wv[T];
  __shared__ float l2c[CH ? D : 1];
  const int tid = threadIdx.x;
  const SeqMap &m = p.m;
  const int H = m.H;
  // (items spread over the XCDs: a head's weighted range is long or short
  // with its decay)
  const int item = xcd_spread((int)blockIdx.x, (int)gridDim.x);
  const int s = item / H, h = item - s * H;
  float log2lam;
  if constexpr (CH) {
    const float *al = p.chdecay + (int64_t)h * D;
    log2lam = -__builtin_huge_valf();
    for (int i = 0; i < D; ++i) log2lam = fmaxf(log2lam, log2f(al[i]));
    for (int i = tid; i < D; i += NT) l2c[i] = log2f(al[i]);
    __syncthreads();
  } else {
    log2lam = log2f(p.decay[h]);
  }
  const int64_t a = (int64_t)s * p.seg_len;
  const int64_t b = (a + p.seg_len < m.total) ? a + p.seg_len : m.total;
  if (a >= b) return;
  const int jl = m.seq_of(b - 1);
  // A segment whose last piece ends its sequence hands no state onward: the
  // scan never uses its local state.
  if (m.start(jl + 1) == b) return;
  const int64_t ps0 = m.start(jl);
  const int64_t ps = ps0 > a ? ps0 : a;
  const int64_t base = m.row_base(h, jl);
  constexpr int PER = D * D / NT;
  float acc[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) acc[u] = 0.f;
  for (int64_t t0 = first_weighted(ps, b, log2lam, T); t0 < b; t0 += T) {
    const int L = (int)((b - t0) < T ? (b - t0) : T);
    load_rows<Tin, D>(Ks, (const Tin *)p.k + base + t0 * m.rs, m.rs, L, tid);
    load_rows<Tin, D>(Vs, (const Tin *)p.v + base + t0 * m.rs, m.rs, L, tid);
    if constexpr (CH) {
      for (int e = tid; e < T * D; e += NT) {
        const int c = e / D, i = e - (e / D) * D;
        Ks[c][i] = c < L ? Ks[c][i] * pow_lam(l2c[i], (float)(b - 1 - t0 - c)) : 0.f;
      }
      if (tid < T) wv[tid] = 1.f;
    } else {
      if (tid < T) wv[tid] = tid < L ? pow_lam(log2lam, (float)(b - 1 - t0 - tid)) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      int e = u * NT + tid, i = e / D, j = e - (e / D) * D;
      float sacc = 0.f;
      for (int c = 0; c < L; ++c) sacc += (wv[c] * Ks[c][i]) * Vs[c][j];
      acc[u] += sacc;
    }
    __syncthreads();
  }
  float *dst = p.ws + ((int64_t)s * H + h) * (int64_t)D * D;
#pragma unroll
  for (int u = 0; u < PER; ++u) dst[u * NT + tid] = acc[u];
}

}  // namespace simt
}  // namespace la
