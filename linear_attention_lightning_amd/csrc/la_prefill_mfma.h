// bf16 prefill on gfx950 MFMA (v_mfma_f32_32x32x16_bf16), d = 128.
//
// One workgroup (4 waves) owns one (segment, head).  It walks the segment in
// chunks of at most 128 tokens, carrying the 128 x 128 float32 state in MFMA
// accumulators spread over the 4 waves (wave w owns state rows 32w..32w+31).
// Per chunk (MiniMax-01 report, section 2.2.1: left product inside the
// block, right product between blocks), with L rows, a_r = lambda^(r+1),
// D_rc = lambda^(r-c) for r >= c, b_c = lambda^(L-1-c):
//     O^T = diag(a) (S^T Q^T)  +  V^T ((K Q^T) (.) D^T)      (wave w: rows 32w..)
//     S   = lambda^L S + (diag(b) K)^T V
// Everything is computed transposed so that the query row is each lane's
// fixed MFMA column: the K Q^T accumulator then feeds the next MFMA as its B
// operand straight from registers (its row groups of 4 consecutive keys are
// the k slots, read in the same order from V by ds_read_b64_tr_b16), the
// decay scale a_r is one value per lane, and the output leaves as 8-byte
// stores of 4 consecutive features.
//
// MFMA 32x32x16 operand layout (lane l, l32 = l % 32, g = l / 32):
//   A[m][k]: lane holds m = l32, k = 8g .. 8g+7
//   B[k][n]: lane holds n = l32, k = 8g .. 8g+7
//   D[m][n]: lane holds n = l32, register r holds m = 8(r/4) + 4g + r%4
// ds_read_b64_tr_b16: in each 16-lane group, lane i16 supplies the address
// of 4 consecutive 16-bit elements of row (i16 / 4), columns 4 (i16 % 4)..;
// lane i16 receives element (row e, column i16) for e = 0..3.
#pragma once

#include "la_common.h"

namespace la {
namespace mfma {

constexpr int D = 128;
constexpr int T = 128;          // tokens per chunk
constexpr int NT = 256;         // threads per workgroup
constexpr int RSQ = 2 * D + 16; // LDS row stride (bytes) of Q and S^T tiles
constexpr int RSK = 2 * D + 32; // LDS row stride (bytes) of K and V tiles
constexpr int LDS_Q = T * RSQ;
constexpr int LDS_K = T * RSK;
constexpr int LDS_ST = D * RSQ;
constexpr int LDS_BYTES = LDS_Q + 2 * LDS_K + LDS_ST;

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two transposed LDS reads: rows r0..r0+3 and r0+off..r0+off+3 of a row-major
// bf16 tile, the lane's column; p is this lane's address for the first read.
__device__ __forceinline__ bf16x8 tr_read8(const char *p, int off_bytes) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LA_LDS s16x4 *)(p));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LA_LDS s16x4 *)(p + off_bytes));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ bf16x8 cvt8(float a0, float a1, float a2, float a3, float a4, float a5,
                                       float a6, float a7) {
  bf16x8 r = {(bf16)a0, (bf16)a1, (bf16)a2, (bf16)a3, (bf16)a4, (bf16)a5, (bf16)a6, (bf16)a7};
  return r;
}

// Global -> registers: rows [0, L) of a 128 x 128 bf16 tile starting at src;
// rows >= L read as zero.  Thread t moves 16 bytes of row (it*256 + t)/16.
__device__ __forceinline__ void load_tile(uint4 (&r)[8], const bf16 *src, int L, int tid) {
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    int id = it * NT + tid, row = id >> 4, c16 = id & 15;
    if (row < L) r[it] = *(const uint4 *)(src + (int64_t)row * D + c16 * 8);
    else r[it] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void store_tile_lds(char *dst, int rs, const uint4 (&r)[8], int tid) {
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    int id = it * NT + tid, row = id >> 4, c16 = id & 15;
    *(uint4 *)(dst + row * rs + c16 * 16) = r[it];
  }
}

// State accumulators: S[nt] register r of lane (l32, g) in wave w holds
// S[i][j] with i = 32w + 8(r/4) + 4g + r%4 and j = 32 nt + l32.
__device__ __forceinline__ void load_state(f32x16 (&S)[4], const float *src, int w, int l32,
                                           int g) {
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int i = 32 * w + 8 * (r >> 2) + 4 * g + (r & 3), j = 32 * nt + l32;
      S[nt][r] = src ? src[i * D + j] : 0.f;
    }
}

__device__ __forceinline__ void store_state(float *dst, const f32x16 (&S)[4], int w, int l32,
                                            int g) {
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int i = 32 * w + 8 * (r >> 2) + 4 * g + (r & 3), j = 32 * nt + l32;
      dst[i * D + j] = S[nt][r];
    }
}

// S^T (bf16) into LDS: row j holds S[0..127][j].
__device__ __forceinline__ void write_st(char *STs, const f32x16 (&S)[4], int w, int l32, int g) {
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      bf16x4 v = {(bf16)S[nt][4 * rq], (bf16)S[nt][4 * rq + 1], (bf16)S[nt][4 * rq + 2],
                  (bf16)S[nt][4 * rq + 3]};
      *(bf16x4 *)(STs + (32 * nt + l32) * RSQ + (32 * w + 8 * rq + 4 * g) * 2) = v;
    }
}

// S += (diag(wgt) K)^T V over the chunk in LDS, wgt_c = 2^(e0 - c) log2lam)
// for c < L and 0 otherwise (e0 = L - 1 inside a block; the distance to the
// segment's last token in the local-state pass).
__device__ __forceinline__ void state_update(f32x16 (&S)[4], const char *Ks, const char *Vs,
                                             int L, float e0, float log2lam, int w, int lane) {
  const int g = lane >> 5, G16 = lane >> 4, i16 = lane & 15;
  const int sub = (i16 >> 2) * RSK + (16 * (G16 & 1) + 4 * (i16 & 3)) * 2;
#pragma unroll 2
  for (int ks = 0; ks < T / 16; ++ks) {
    const int c0 = 16 * ks + 8 * g;
    bf16x8 kf = tr_read8(Ks + c0 * RSK + (32 * w) * 2 + sub, 4 * RSK);
    float wv[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      int c = c0 + s;
      wv[s] = c < L ? pow_lam(log2lam, e0 - (float)c) * (float)kf[s] : 0.f;
    }
    bf16x8 a = cvt8(wv[0], wv[1], wv[2], wv[3], wv[4], wv[5], wv[6], wv[7]);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      bf16x8 b = tr_read8(Vs + c0 * RSK + (32 * nt) * 2 + sub, 4 * RSK);
      S[nt] = mma(a, b, S[nt]);
    }
  }
}

// Phase C: outputs (and final states) for one (segment, head).
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_chunk_kernel(FwdArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  char *Qs = smem, *Ks = smem + LDS_Q, *Vs = Ks + LDS_K, *STs = Vs + LDS_K;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5, G16 = lane >> 4, i16 = lane & 15;
  const SeqMap &m = p.m;
  const int H = m.H;
  const int s = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const float log2lam = log2f(p.decay[h]);
  const int64_t a = (int64_t)s * p.seg_len;
  const int64_t b = (a + p.seg_len < m.total) ? a + p.seg_len : m.total;
  const int64_t DD = (int64_t)D * D;

  Cursor cur = first_chunk(m, a, b, T);
  if (!cur.valid) return;

  f32x16 S[4];
  {
    const float *s0 = p.ws ? p.ws + ((int64_t)s * H + h) * DD
                           : (p.init ? p.init + ((int64_t)cur.j * H + h) * DD : nullptr);
    load_state(S, s0, w, l32, g);
  }
  uint4 pq[8], pk[8], pv[8];
  {
    const int64_t base = m.row_base(h, cur.j) + cur.c0 * D;
    const int L0 = (int)(cur.c1 - cur.c0);
    load_tile(pq, (const bf16 *)p.q + base, L0, tid);
    load_tile(pk, (const bf16 *)p.k + base, L0, tid);
    load_tile(pv, (const bf16 *)p.v + base, L0, tid);
    store_tile_lds(Qs, RSQ, pq, tid);
    store_tile_lds(Ks, RSK, pk, tid);
    store_tile_lds(Vs, RSK, pv, tid);
    write_st(STs, S, w, l32, g);
  }
  __syncthreads();

  const int row = 32 * w + l32;  // this lane's query row inside the chunk
  const int tr_sub = (i16 >> 2) * RSK + (16 * (G16 & 1) + 4 * (i16 & 3)) * 2;

  while (true) {
    const Cursor nxt = next_chunk(m, cur, b, T);
    if (nxt.valid) {  // prefetch the next chunk while this one computes
      const int64_t base = m.row_base(h, nxt.j) + nxt.c0 * D;
      const int Ln = (int)(nxt.c1 - nxt.c0);
      load_tile(pq, (const bf16 *)p.q + base, Ln, tid);
      load_tile(pk, (const bf16 *)p.k + base, Ln, tid);
      load_tile(pv, (const bf16 *)p.v + base, Ln, tid);
    }
    const int L = (int)(cur.c1 - cur.c0);

    // Q^T fragments of this wave's 32 query rows (B operand, k = feature).
    bf16x8 qf[8];
    {
      const char *qrow = Qs + row * RSQ + 16 * g;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8 *)(qrow + 32 * ks);
    }
    // Inter-block term: O^T = S^T Q^T, then scaled by a_row = lambda^(row+1).
    f32x16 acc[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      acc[jt] = (f32x16){};
      const char *strow = STs + (32 * jt + l32) * RSQ + 16 * g;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) acc[jt] = mma(*(const bf16x8 *)(strow + 32 * ks), qf[ks], acc[jt]);
      acc[jt] *= pow_lam(log2lam, (float)(row + 1));
    }
    // Intra-block term over key sub-blocks kc <= w (causal).
    for (int kc = 0; kc <= w; ++kc) {
      f32x16 pt = {};
      const char *krow = Ks + (32 * kc + l32) * RSK + 16 * g;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) pt = mma(*(const bf16x8 *)(krow + 32 * ks), qf[ks], pt);
      // pt register r: key c = 32kc + 8(r/4) + 4g + r%4, query `row`.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int c = 32 * kc + 8 * (r >> 2) + 4 * g + (r & 3);
        pt[r] = (c <= row) ? pt[r] * pow_lam(log2lam, (float)(row - c)) : 0.f;
      }
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        bf16x8 pb = cvt8(pt[8 * q2], pt[8 * q2 + 1], pt[8 * q2 + 2], pt[8 * q2 + 3],
                         pt[8 * q2 + 4], pt[8 * q2 + 5], pt[8 * q2 + 6], pt[8 * q2 + 7]);
        const int c0 = 32 * kc + 16 * q2 + 4 * g;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          bf16x8 vf = tr_read8(Vs + c0 * RSK + (32 * jt) * 2 + tr_sub, 8 * RSK);
          acc[jt] = mma(vf, pb, acc[jt]);
        }
      }
    }
    // Store: acc[jt] registers 4rq..4rq+3 hold features 32jt + 8rq + 4g + 0..3.
    if (row < L) {
      bf16 *orow = (bf16 *)p.out + m.row_base(h, cur.j) + (cur.c0 + row) * D;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          bf16x4 v = {(bf16)acc[jt][4 * rq], (bf16)acc[jt][4 * rq + 1], (bf16)acc[jt][4 * rq + 2],
                      (bf16)acc[jt][4 * rq + 3]};
          *(bf16x4 *)(orow + 32 * jt + 8 * rq + 4 * g) = v;
        }
    }
    // State after this chunk, when anything still needs it.
    const bool seq_done = (cur.c1 == cur.seq_end);
    const bool new_piece = nxt.valid && (nxt.c0 >= cur.pend);
    if ((nxt.valid && !new_piece) || (seq_done && p.fin)) {
      const float gL = pow_lam(log2lam, (float)L);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) S[nt] *= gL;
      state_update(S, Ks, Vs, L, (float)(L - 1), log2lam, w, lane);
      if (seq_done && p.fin) store_state(p.fin + ((int64_t)cur.j * H + h) * DD, S, w, l32, g);
    }
    if (!nxt.valid) break;
    if (new_piece)
      load_state(S, p.init ? p.init + ((int64_t)nxt.j * H + h) * DD : nullptr, w, l32, g);
    __syncthreads();  // every wave is done with this chunk's LDS tiles
    store_tile_lds(Qs, RSQ, pq, tid);
    store_tile_lds(Ks, RSK, pk, tid);
    store_tile_lds(Vs, RSK, pv, tid);
    write_st(STs, S, w, l32, g);
    __syncthreads();
    cur = nxt;
  }
}

// Phase A: the local state of each segment's last piece, from zero:
//   L_s = sum_{c in [ps, b)} lambda^(b-1-c) k_c^T v_c.
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void local_state_kernel(FwdArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * LDS_K];
  char *Ks = smem, *Vs = smem + LDS_K;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const SeqMap &m = p.m;
  const int H = m.H;
  const int s = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const float log2lam = log2f(p.decay[h]);
  const int64_t a = (int64_t)s * p.seg_len;
  const int64_t b = (a + p.seg_len < m.total) ? a + p.seg_len : m.total;
  if (a >= b) return;
  const int jl = m.seq_of(b - 1);
  const int64_t ps0 = m.start(jl);
  const int64_t ps = ps0 > a ? ps0 : a;
  const int64_t base = m.row_base(h, jl);

  f32x16 S[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) S[nt] = (f32x16){};
  uint4 pk[8], pv[8];
  int L = (int)((b - ps) < T ? (b - ps) : T);
  load_tile(pk, (const bf16 *)p.k + base + ps * D, L, tid);
  load_tile(pv, (const bf16 *)p.v + base + ps * D, L, tid);
  for (int64_t t0 = ps; t0 < b; t0 += T) {
    store_tile_lds(Ks, RSK, pk, tid);
    store_tile_lds(Vs, RSK, pv, tid);
    __syncthreads();
    const int Lc = L;
    const int64_t t1 = t0 + T;
    if (t1 < b) {
      L = (int)((b - t1) < T ? (b - t1) : T);
      load_tile(pk, (const bf16 *)p.k + base + t1 * D, L, tid);
      load_tile(pv, (const bf16 *)p.v + base + t1 * D, L, tid);
    }
    // weight of chunk row c: lambda^(b - 1 - (t0 + c))
    state_update(S, Ks, Vs, Lc, (float)(b - 1 - t0), log2lam, w, lane);
    __syncthreads();
  }
  store_state(p.ws + ((int64_t)s * H + h) * (int64_t)D * D, S, w, l32, g);
}

}  // namespace mfma
}  // namespace la
