// bf16 prefill on gfx950 MFMA (v_mfma_f32_16x16x32_bf16 and 32x32x16), d = 128.
//
// One workgroup owns one (segment, head) and walks it in chunks of at most
// 128 tokens (MiniMax-01 report, section 2.2.1: left product inside a block,
// right product between blocks, the block state carried forward).  Per chunk
// with L rows, a_r = lambda^(r+1), D_rc = lambda^(r-c) (r >= c),
// b_c = lambda^(L-1-c):
//     O^T = diag(a) (S^T Q^T)  +  V^T ((K Q^T) (.) D^T)
//     S   = lambda^L S + (diag(b) K)^T V
// The workgroup has 8 waves in two roles that run side by side, with two
// barriers per chunk: A opens it (its K/V tiles and the S^T of the state
// entering it are in LDS), B closes it (every read of those is done).
//   output waves 0-3: wave w owns the 16-row query blocks w and 7 - w (the
//     same causal work for every wave) and runs 16x16x32 MFMAs; its Q^T
//     fragments come straight from HBM into registers a chunk ahead.  After
//     A it computes the inter-block term from the published S^T, then the
//     intra-block term (the key steps both blocks share read each K and V
//     fragment once for both); after B it stages its rows in the chunk's
//     now free K tile and writes them back as whole 256-byte rows.
//   state waves 4-7: wave 4+u owns state rows 32u..32u+31 in float32
//     32x32x16 MFMA accumulators.  After A they update the state, issuing
//     the next chunk's K/V tiles HBM -> LDS by DMA (global_load_lds, no
//     registers) as they go; after B they publish the new state as bf16 S^T
//     and wait for the next tiles to land.
// Everything is computed transposed so the query row is each lane's fixed
// MFMA column: the K Q^T accumulator (register quads hold 4 consecutive
// keys) feeds V^T (K Q^T) directly as the B operand, with V read in the same
// key order by ds_read_b64_tr_b16; a_r is one scalar per lane.
//
// MFMA 32x32x16 operand layout (lane l, l32 = l % 32, g = l / 32):
//   A[m][k]: lane holds m = l32, k = 8g .. 8g+7
//   B[k][n]: lane holds n = l32, k = 8g .. 8g+7
//   D[m][n]: lane holds n = l32, register r holds m = 8(r/4) + 4g + r%4
// ds_read_b64_tr_b16: in each 16-lane group, lane i16 supplies the address
// of 4 consecutive 16-bit elements of row (i16 / 4), columns 4 (i16 % 4)..;
// lane i16 receives element (row e, column i16) for e = 0..3.
//
// Powers of lambda: 2^(n log2 lambda) on v_exp_f32, factored as one
// exponential per register quad times per-lane constants lambda^0..lambda^7
// when lambda > 2^-15 (so no factor can overflow); below that every power is
// exponentiated on its own.
#pragma once

#include <type_traits>

#include "la_common.h"

namespace la {
namespace mfma {

// Phase timing of the chunk kernel (built only with -DLA_PHASE_PROBE, by
// phase_probe.py; the library itself has no such code): lane 0 of output
// wave 0 and of state wave 4 records the shader clock (s_memtime) at the
// barriers and phase ends of each chunk, for the first 256 workgroups and
// 64 chunks of a launch, at [workgroup][chunk][slot].
// The local-state pass likewise: thread 0 of each of the first 1024
// workgroups, at the steps of its first 40 chunks, at [workgroup][chunk][slot].
#ifdef LA_PHASE_PROBE
__device__ unsigned long long g_phase_probe[256 * 64 * 16];
__device__ unsigned long long g_phase_probe_local[1024 * 40 * 4];
#endif
__device__ __forceinline__ void phase_mark(bool on, int ci, int slot, int lane) {
#ifdef LA_PHASE_PROBE
  const unsigned long long t = __builtin_amdgcn_s_memtime();
  const int bid = blockIdx.x;
  if (on && lane == 0 && bid < 256 && ci < 64) g_phase_probe[(bid * 64 + ci) * 16 + slot] = t;
#else
  (void)on, (void)ci, (void)slot, (void)lane;
#endif
}
__device__ __forceinline__ void phase_mark_local(bool on, int ci, int slot, int tid) {
#ifdef LA_PHASE_PROBE
  const unsigned long long t = __builtin_amdgcn_s_memtime();
  const int bid = blockIdx.x;
  if (on && tid == 0 && bid < 1024 && ci < 40) g_phase_probe_local[(bid * 40 + ci) * 4 + slot] = t;
#else
  (void)on, (void)ci, (void)slot, (void)tid;
#endif
}

constexpr int D = 128;
constexpr int T = 128;           // tokens per chunk
constexpr int NT = 512;          // threads per workgroup of the chunk kernel (8 waves)
constexpr int NT_LOCAL = 256;    // threads per workgroup of the local-state kernel
constexpr int C_LOCAL = 64;      // tokens per chunk of the local-state kernel
constexpr int KV_ROW = 2 * D;      // LDS row stride (bytes) of every 128 x 128 bf16 tile
constexpr int LDS_K = T * KV_ROW;  // one K or V tile (32 KB, swizzled)
constexpr int LDS_KV = 2 * LDS_K;  // the K and V tiles of one chunk
constexpr int LDS_ST = D * KV_ROW; // S^T (32 KB, swizzled like the tiles)
// Cache-policy operand of a buffer access: the non-temporal hint (CDNA3/4
// "nt", the SLC bit of the encoding).  q, k, v and out are each touched once
// per pass, so the streaming accesses of the output pass (Q loads, K/V tile
// loads, output stores) carry it: measured 7-8% less time per headline step
// than cached accesses.
constexpr int kCpolNT = 2;
// The chunk kernel: two chunks' K/V tiles (double buffer) and S^T: 160 KB.
constexpr int LDS_BYTES = 2 * LDS_KV + LDS_ST;
constexpr float kFastLog2 = -15.f;  // factored powers when log2(lambda) > this
// Word 3 of a raw (unswizzled, stride 0) buffer resource on gfx9-family
// GPUs: 32-bit data format, no index addressing; an access at or past the
// resource's byte range reads zero or writes nothing.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// K and V tiles: 128 rows of 256 bytes, unpadded; the 16-byte granule c of
// row r is stored at granule c ^ kv_swz(r).  With this permutation every
// access pattern used on the tiles reaches each of the 64 LDS banks once per
// cycle (measured on gfx950: a row-per-lane 16-byte read runs at 5 clocks
// per wave instruction instead of 8.5 with 288-byte rows, the transposed
// read at 3 instead of 4.6):
//   16 lanes reading one granule of 16 consecutive rows (MFMA A operand);
//   ds_read_b64_tr_b16 over rows 4m..4m+3 and one 64-byte column block;
//   16 lanes writing one whole row.
// kv_swz depends on r mod 16 only, so adding 16 rows is adding 4096 bytes.
__device__ __forceinline__ int kv_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int kv_off(int r, int byte) {
  return r * KV_ROW + ((((byte >> 4) ^ kv_swz(r)) << 4) | (byte & 15));
}

// This lane's address offset for ds_read_b64_tr_b16 over rows r4..r4+3
// (r4 a multiple of 4) and columns 32 blk .. 32 blk + 31 of a K/V tile: in
// each 16-lane group, lane i16 points at 4 consecutive elements of row
// r4 + i16/4, columns 32 blk + 16 (G16 & 1) + 4 (i16 & 3) ...
__device__ __forceinline__ int tr_off(int r4, int blk, int G16, int i16) {
  return kv_off(r4 + (i16 >> 2), 64 * blk + 32 * (G16 & 1) + 8 * (i16 & 3));
}

// Two transposed LDS reads of a K/V tile at this lane's offsets o0 and o1
// (two groups of 4 rows, the lane's column); base may add a multiple of 16
// rows.
__device__ __forceinline__ bf16x8 tr_read8(const char *base, int o0, int o1) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LA_LDS s16x4 *)(base + o0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LA_LDS s16x4 *)(base + o1));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// 32-bit LDS byte addresses.  The swizzle only permutes bits 4..7 of a
// tile offset, so for a tile base aligned to 256 bytes, kv_off(r, B + 16 x)
// = kv_off(r, B) ^ (x << 4) whenever B / 16 and x share no bits: the
// per-fragment addresses of the output side are formed as one XOR of a
// per-chunk base (which keeps the compiler from hoisting dozens of
// loop-invariant offsets into registers).
__device__ __forceinline__ unsigned lds_u32(const char *p) {
  return (unsigned)(size_t)(const LA_LDS char *)p;
}
template <class T>
__device__ __forceinline__ T lds_ld(unsigned a) {
  return *(const LA_LDS T *)a;
}
template <class T>
__device__ __forceinline__ void lds_st(unsigned a, T v) {
  *(LA_LDS T *)a = v;
}
__device__ __forceinline__ bf16x8 tr_read8u(unsigned a0, unsigned a1) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LA_LDS s16x4 *)a0);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LA_LDS s16x4 *)a1);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ bf16x8 cvt8(const float (&v)[8]) {
  bf16x8 r = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3],
              (bf16)v[4], (bf16)v[5], (bf16)v[6], (bf16)v[7]};
  return r;
}

// FwdArgs::flags of the gated path: the normalisation, SiLU activation and
// gate the MiniMax-01 report places around its attention and leaves out of
// its derivation (section 2.2.1).  The reading computed here, each part
// selected by a flag: SiLU(x) = x / (1 + e^-x) on q, k and/or v as they are
// read; RMS normalisation of every output row over the head's 128 channels,
// o / sqrt(mean(o^2) + eps), times a per-channel weight [H][128]; an output
// gate o * sigmoid(g), g laid out like the output.  The normalisation runs on
// the float32 accumulators, weight and gate on the row as it is stored.
enum : int { GF_SILU_Q = 1, GF_SILU_K = 2, GF_SILU_V = 4, GF_NORM = 8, GF_GATE = 16 };

constexpr float kLog2e = 1.4426950408889634f;

// x / (1 + e^-x) for each of 8 bf16 values, in float32, rounded to bf16.
__device__ __forceinline__ u32x4 silu8(u32x4 x) {
  const bf16x8 v = __builtin_bit_cast(bf16x8, x);
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float f = (float)v[e];
    r[e] = f * __builtin_amdgcn_rcpf(1.f + fast_exp2(-f * kLog2e));
  }
  return __builtin_bit_cast(u32x4, cvt8(r));
}

// Global -> registers: a 128 x 128 bf16 tile whose row i starts at
// src + i * rs, of which rows [0, L) are valid (L >= 1), moved by `nthr`
// threads (thread t of them moves 16 bytes of row (it * nthr + t) / 16).  Rows >= L repeat row L - 1: every
// consumer masks those rows out or multiplies them by exact zeros, so any
// finite values do, and the loads need no branches (a branch around a load
// makes the compiler's memory-wait analysis far more conservative).
template <int NTHR, int ROWS = T>
__device__ __forceinline__ void load_tile(u32x4 (&r)[ROWS * 16 / NTHR], const bf16 *src,
                                          int64_t rs, int L, int t) {
#pragma unroll
  for (int it = 0; it < ROWS * 16 / NTHR; ++it) {
    const int id = it * NTHR + t, row = id >> 4, c16 = id & 15;
    const int rr = row < L ? row : L - 1;
    r[it] = *(const u32x4 *)(src + (int64_t)rr * rs + c16 * 8);
  }
}

template <int NTHR, int ROWS = T>
__device__ __forceinline__ void store_tile(char *dst, const u32x4 (&r)[ROWS * 16 / NTHR], int t) {
#pragma unroll
  for (int it = 0; it < ROWS * 16 / NTHR; ++it) {
    int id = it * NTHR + t, row = id >> 4, c16 = id & 15;
    *(u32x4 *)(dst + kv_off(row, c16 * 16)) = r[it];
  }
}

// State accumulators: S[nt] register r of lane (l32, g) in the wave owning
// rows 32u.. holds S[i][j], i = 32u + 8(r/4) + 4g + r%4, j = 32 nt + l32.
// One base pointer per register quad; the rest of every element's offset,
// (r%4) D + 32 nt floats, fits the instructions' immediate offset field, so
// the 64 accesses need only four address registers.
__device__ __forceinline__ void load_state(f32x16 (&S)[4], const float *src, int u, int l32,
                                           int g) {
  if (!src) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[nt] = (f32x16){};
    return;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float *bq = src + (32 * u + 8 * q + 4 * g) * D + l32;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) S[nt][4 * q + mm] = bq[mm * D + 32 * nt];
  }
}

__device__ __forceinline__ void store_state(float *dst, const f32x16 (&S)[4], int u, int l32,
                                            int g) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float *bq = dst + (32 * u + 8 * q + 4 * g) * D + l32;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) bq[mm * D + 32 * nt] = S[nt][4 * q + mm];
  }
}

// S^T (bf16) into LDS, swizzled like the K/V tiles: row j holds S[0..127][j].
__device__ __forceinline__ void write_st(char *STs, const f32x16 (&S)[4], int u, int l32, int g) {
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      bf16x4 v = {(bf16)S[nt][4 * rq], (bf16)S[nt][4 * rq + 1], (bf16)S[nt][4 * rq + 2],
                  (bf16)S[nt][4 * rq + 3]};
      *(bf16x4 *)(STs + kv_off(32 * nt + l32, (32 * u + 8 * rq + 4 * g) * 2)) = v;
    }
}

// S += (diag(wgt) K)^T V over the first 16 NKS rows of the tile in LDS, for
// this wave's state rows 32u..32u+31: wgt_c = lambda^(e0 - c) for chunk rows
// c < L, else 0.
// tail8[s] = lambda^(7 - s) (fast path only).
struct NoHook {
  __device__ __forceinline__ void operator()(int) const {}
};

// hook(ks) runs at the start of step ks (PIPE path): the chunk loop issues
// the next chunk's tile loads there, spread over the update.
template <int NKS = T / 16, bool PIPE = true, typename Hook = NoHook>
__device__ __forceinline__ void state_update(f32x16 (&S)[4], const char *Ks, const char *Vs,
                                             int L, int e0, float l2, bool fast,
                                             const float (&tail8)[8], int u, int lane,
                                             const Hook &hook = Hook()) {
  const int g = lane >> 5, G16 = lane >> 4, i16 = lane & 15;
  // Rows 16 ks + 8 g + (0..3, 4..7): K columns 32u.., V columns 32 nt..
  const int ko0 = tr_off(8 * g, u, G16, i16), ko1 = tr_off(8 * g + 4, u, G16, i16);
  int vo0[4], vo1[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    vo0[nt] = tr_off(8 * g, nt, G16, i16);
    vo1[nt] = tr_off(8 * g + 4, nt, G16, i16);
  }
  // A operand of step ks: the weighted K^T fragment.
  auto weighted = [&](bf16x8 kf, int ks) -> bf16x8 {
    const int c0 = 16 * ks + 8 * g;
    float wv[8];
    if (fast) {
      const float e = fast_exp2((float)(e0 - c0 - 7) * l2);
#pragma unroll
      for (int s = 0; s < 8; ++s) wv[s] = (c0 + s < L) ? (float)kf[s] * (e * tail8[s]) : 0.f;
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s)
        wv[s] = (c0 + s < L) ? (float)kf[s] * fast_exp2((float)(e0 - c0 - s) * l2) : 0.f;
    }
    return cvt8(wv);
  };
  if constexpr (PIPE) {
    // Software-pipelined: the LDS reads of step ks + 1 go out before the
    // arithmetic and MFMAs of step ks, so their latency overlaps work.
    bf16x8 kf[2], vf[2][4];
    auto fetch = [&](int ks, int slot) {
      kf[slot] = tr_read8(Ks + 16 * ks * KV_ROW, ko0, ko1);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        vf[slot][nt] = tr_read8(Vs + 16 * ks * KV_ROW, vo0[nt], vo1[nt]);
    };
    fetch(0, 0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int sl = ks & 1;
      if (ks + 1 < NKS) fetch(ks + 1, sl ^ 1);
      hook(ks);
      const int c0 = 16 * ks + 8 * g;
      float wv[8];
      if (fast) {
        const float e = fast_exp2((float)(e0 - c0 - 7) * l2);
#pragma unroll
        for (int s = 0; s < 8; ++s) wv[s] = (c0 + s < L) ? (float)kf[sl][s] * (e * tail8[s]) : 0.f;
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s)
          wv[s] = (c0 + s < L) ? (float)kf[sl][s] * fast_exp2((float)(e0 - c0 - s) * l2) : 0.f;
      }
      const bf16x8 a = cvt8(wv);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) S[nt] = mma(a, vf[sl][nt], S[nt]);
    }
  } else {
    // Fewer registers (for kernels that run several workgroups per CU).
#pragma unroll 2
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 a = weighted(tr_read8(Ks + 16 * ks * KV_ROW, ko0, ko1), ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        S[nt] = mma(a, tr_read8(Vs + 16 * ks * KV_ROW, vo0[nt], vo1[nt]), S[nt]);
    }
  }
}

__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Inter-block term O^T = S^T Q^T for the wave's two 16-row query blocks,
// block bi scaled by a[bi] = lambda^(row + 1) of this lane's query row.
// acc[bi][jt] register r: feature 16 jt + 4 G + r of the lane's query.  One
// S^T fragment (rows 16 jt + i16, features 32 ks + 8 G ..) serves both
// blocks; st = LDS address of S^T + kv_off(i16, 16 G), so fragment (jt, ks)
// sits at (st ^ (ks << 6)) + 4096 jt.
__device__ __forceinline__ void inter_term(f32x4 (&acc)[2][8], unsigned st,
                                           const u32x4 (&qf)[2][4], const float (&a)[2]) {
  // Software-pipelined one feature tile ahead; the scheduling barriers keep
  // the compiler from hoisting every tile's reads (128 registers) up front.
  bf16x8 sf[2][4];
  auto fetch = [&](int jt, int slot) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) sf[slot][ks] = lds_ld<bf16x8>((st ^ (ks << 6)) + 4096 * jt);
  };
  fetch(0, 0);
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) {
    if (jt + 1 < 8) fetch(jt + 1, (jt + 1) & 1);
    acc[0][jt] = (f32x4){};
    acc[1][jt] = (f32x4){};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      acc[0][jt] = mma16(sf[jt & 1][ks], as_bf16x8(qf[0][ks]), acc[0][jt]);
      acc[1][jt] = mma16(sf[jt & 1][ks], as_bf16x8(qf[1][ks]), acc[1][jt]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) {
    acc[0][jt] *= a[0];
    acc[1][jt] *= a[1];
    // Materialise the results here: left alone, the compiler sinks block 1's
    // products past block 0's intra-block loop (to where they are first
    // needed) and keeps the S^T fragments alive across it.
    asm volatile("" : "+v"(acc[0][jt]), "+v"(acc[1][jt]));
  }
}

// The same product with the published tile read transposed: the tile holds
// M^T (row j = column j of M, as write_st lays out S^T) and the A operand is
// M itself, so this is O^T = M Q^T for the state M = S^T.  Fragment (jt, ks)
// of M (rows 16 jt + i16, columns 32 ks + 8 G ..) is column 16 jt + i16 of
// tile rows 32 ks + 8 G + (0..7): two ds_read_b64_tr_b16 over rows
// 32 ks + 8 G + (0..3) and + (4..7), at (t0 + 8192 ks) ^ (jt << 5) and
// (t1 + 8192 ks) ^ (jt << 5), where t0 and t1 are the tile's LDS address plus
// kv_off(8 G + i16 / 4, 8 (i16 % 4)) and kv_off(8 G + 4 + i16 / 4, ..).
__device__ __forceinline__ void inter_term_tr(f32x4 (&acc)[2][8], unsigned t0, unsigned t1,
                                              const u32x4 (&qf)[2][4], const float (&a)[2]) {
  bf16x8 sf[2][4];
  auto fetch = [&](int jt, int slot) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      sf[slot][ks] = tr_read8u((t0 + 8192 * ks) ^ (jt << 5), (t1 + 8192 * ks) ^ (jt << 5));
  };
  fetch(0, 0);
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) {
    if (jt + 1 < 8) fetch(jt + 1, (jt + 1) & 1);
    acc[0][jt] = (f32x4){};
    acc[1][jt] = (f32x4){};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      acc[0][jt] = mma16(sf[jt & 1][ks], as_bf16x8(qf[0][ks]), acc[0][jt]);
      acc[1][jt] = mma16(sf[jt & 1][ks], as_bf16x8(qf[1][ks]), acc[1][jt]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) {
    acc[0][jt] *= a[0];
    acc[1][jt] *= a[1];
    asm volatile("" : "+v"(acc[0][jt]), "+v"(acc[1][jt]));
  }
}

// Per-workgroup constants and lane coordinates of the 8-wave layout.  The
// wave index lives in a scalar register, so the role test is a scalar branch
// and each role runs a loop of its own.  (With one exec-masked instruction
// stream for both roles, the compiler's memory-wait analysis sees the other
// role's loads into the same registers and waits for every prefetch right
// after issuing it.)
struct Lanes {
  int tid, lane, wave, w, l32, g, G16, i16, ts;
  bool out_wave;
  __device__ __forceinline__ Lanes() {
    tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    out_wave = wave < 4;
    w = wave & 3;  // output query blocks w and 7 - w, or state rows 32w..
    l32 = lane & 31;
    g = lane >> 5;
    G16 = lane >> 4;
    i16 = lane & 15;
    ts = tid - 256;  // state waves: index among the 256 loaders
  }
  // Output waves: query block bi (0: rows 16w.., 1: rows 16(7-w)..).
  __device__ __forceinline__ int qblock(int bi) const { return bi ? 7 - w : w; }
};

struct Decay {
  float l2;       // log2(lambda), uniform
  bool fast;      // factored powers allowed
  float tail[8];  // lambda^(7-s), s = 0..7 (also lambda^(3-m) = tail[4+m])
  __device__ __forceinline__ explicit Decay(float lam) {
    l2 = uniform(log2f(lam));
    fast = l2 > kFastLog2;
#pragma unroll
    for (int i = 0; i < 8; ++i) tail[i] = uniform(fast_exp2((float)(7 - i) * l2));
  }
};

// Lane coordinates of an output wave (query blocks w and 7 - w), derived
// from the lane id after it passes through an empty asm statement.  Built
// afresh where the chunk loop needs them, so the compiler cannot hoist the
// derived offsets and row numbers out of the loop and keep a dozen more
// registers alive across it.
struct OutLane {
  int lane, i16, G, w;
  __device__ __forceinline__ OutLane(int lane_id, int wave) {
    int l = lane_id;
    asm volatile("" : "+v"(l));
    lane = l;
    i16 = l & 15;
    G = l >> 4;
    w = wave;
  }
  __device__ __forceinline__ int qblock(int bi) const { return bi ? 7 - w : w; }
};

// Q^T fragments of chunk c for query block bi of this output wave, straight
// from HBM (B operand of the 16x16x32 products: qf[ks] holds features
// 32 ks + 8 G .. + 7 of query row 16 qblock(bi) + i16).  Non-temporal loads.
template <bool REV = false>
__device__ __forceinline__ void issue_q_loads(const FwdArgs &p, int h, const Cursor &c, int bi,
                                              u32x4 (&qf)[4], const OutLane &o) {
  // Rows past the chunk's end read its last row: their outputs are never stored.
  const int Lc = (int)(c.c1 - c.c0);
  const int row = 16 * o.qblock(bi) + o.i16;
  const bf16 *qrow = (const bf16 *)p.q + chunk_row_base<REV>(p.m, h, c) +
                     (c.c0 + (row < Lc ? row : Lc - 1)) * p.m.rs + 8 * o.G;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = __builtin_nontemporal_load((const u32x4 *)(qrow + 32 * ks));
}

// K and V rows of chunk c, spread over the 256 threads of a role (register
// path, used by the single-pass kernel's local-state pass).
__device__ __forceinline__ void issue_kv_loads(const FwdArgs &p, int h, const Cursor &c,
                                               u32x4 (&pk)[8], u32x4 (&pv)[8], const Lanes &ln) {
  const int Lc = (int)(c.c1 - c.c0);
  const int64_t base = p.m.row_base<false>(h, c.j) + c.c0 * p.m.rs;
  load_tile<256>(pk, (const bf16 *)p.k + base, p.m.rs, Lc, ln.ts);
  load_tile<256>(pv, (const bf16 *)p.v + base, p.m.rs, Lc, ln.ts);
}

// s_waitcnt vmcnt(N) (the other counters left alone).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// One global_load_lds_dwordx4 (non-temporal): each lane's 16 bytes at gptr
// land in LDS at lds + 16 x lane.  Issued from inline assembly so that the compiler's
// memory-wait analysis does not see an LDS write: it would otherwise wait for
// the load before every later LDS read and every barrier, serialising the
// prefetch.  The caller waits for these loads itself (vm_wait) before the
// barrier that hands the tile to other waves; the compiler's own waits can
// only over-count them, never under-count.
__device__ __forceinline__ void lds_dma16(const void *gptr, const char *lds) {
  const unsigned a = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(const LA_LDS char *)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(gptr), "s"(a)
               : "memory", "m0");
}

// Rows 32u..32u+31 of chunk c's tile of `src` (K or V) straight from HBM into
// the swizzled LDS tile `tile` (global_load_lds_dwordx4: the data bypass the
// registers, each lane's 16 bytes land at the instruction's LDS base + 16 x
// lane).  Lane i of instruction k fills LDS row 4k + i/16, physical granule
// i % 16, so it reads logical granule (i % 16) ^ kv_swz(row).  Rows past the
// chunk's end repeat its last row (finite values that every consumer masks).
// Eight memory instructions per call.
// Instruction k (0..7) of the above: rows 32u + 4k .. 32u + 4k + 3.
template <bool REV = false>
__device__ __forceinline__ void dma_tile_quad(char *tile, const void *src, const FwdArgs &p, int h,
                                              const Cursor &c, int u, int lane, int k) {
  const int Lc = (int)(c.c1 - c.c0);
  const bf16 *base = (const bf16 *)src + chunk_row_base<REV>(p.m, h, c) + c.c0 * p.m.rs;
  const int sub = lane >> 4, pg = lane & 15;
  const int r = 32 * u + 4 * k + sub;
  const int rr = r < Lc ? r : Lc - 1;
  const bf16 *gp = base + (int64_t)rr * p.m.rs + ((pg ^ kv_swz(r)) << 3);
  lds_dma16(gp, tile + (32 * u + 4 * k) * KV_ROW);
}

// lds_dma16 with a uniform base (SGPR pair) and a 32-bit lane offset: the
// address is base + off.  The base is moved to scalar registers explicitly.
__device__ __forceinline__ void lds_dma16_s(const char *base, unsigned off, const char *lds) {
  const unsigned a = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(const LA_LDS char *)lds);
  // (readfirstlane returns int: each half goes through unsigned, or a low
  // word with bit 31 set would sign-extend over the high word)
  const uint64_t bb = (uint64_t)(size_t)base;
  const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(bb >> 32));
  const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)bb);
  const uint64_t sb = (hi << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(off), "s"((const char *)(size_t)sb), "s"(a)
               : "memory", "m0");
}

// Instruction k of dma_tile_quad for a whole chunk of a plain view (positive
// row stride, every row of the tile inside the chunk): `base` points at the
// chunk's first row, row r's 16-byte granules start at byte r * rsb, so a
// lane's address is one 32-bit offset from a uniform base instead of 64-bit
// arithmetic per load.
__device__ __forceinline__ void dma_quad_whole(char *tile, const char *base, int rsb, int u,
                                               int lane, int k) {
  const int sub = lane >> 4, pg = lane & 15;
  const int r = 32 * u + 4 * k + sub;
  lds_dma16_s(base, (unsigned)(r * rsb + ((pg ^ kv_swz(r)) << 4)), tile + (32 * u + 4 * k) * KV_ROW);
}

template <bool REV = false>
__device__ __forceinline__ void dma_tile_rows(char *tile, const void *src, const FwdArgs &p, int h,
                                              const Cursor &c, int u, int lane) {
#pragma unroll
  for (int k = 0; k < 8; ++k) dma_tile_quad<REV>(tile, src, p, h, c, u, lane, k);
}

// Writes this output wave's 32 staged rows of chunk c as whole rows: per
// query block, lane reads 16 bytes of row 16 qblock + 4 it + lane/16 from the
// swizzled staging tile at Os (LDS address, 256-byte aligned; row r0 + 4 it
// sits at (kv_off(r0, .) ^ (it << 4)) + 1024 it) and stores them.  The stores
// go through a buffer resource whose range ends at the chunk's last row:
// the hardware drops those to rows >= the chunk length, so every store is an
// unconditional instruction (a branch around each one would make the
// compiler's memory-wait analysis assume they might not have been issued,
// and wait for them at the next chunk's first Q^T use).
// NEG: the row stride may be negative (a time-reversed view, rows at
// decreasing addresses): the buffer then starts at the chunk's last row, the
// lowest address, and row r sits at byte (L - 1 - r) * |rsb|; rows >= L are
// given the offset 2^31, past the range (below 2^31 bytes), and dropped.
// REV: the view may be a time-reversed packed view (see SeqMap::row_base).
// Gated epilogue (GF_NORM / GF_GATE): before the store, every row is
// multiplied by the head's normalisation weight (wt: this lane's 8 channels
// 8 c16 .., ones without a weight) and by sigmoid of its gate values (gr:
// this lane's 16 bytes of the gate rows written, in write order).
struct Epi {
  float wt[8];
  u32x4 gr[8];
  bool gate;
};

template <bool NEG = false, bool REV = false, bool EPI = false>
__device__ __forceinline__ void write_rows(const FwdArgs &p, int h, const Cursor &c, unsigned Os,
                                           const OutLane &o, const Epi *ep = nullptr) {
  const int L = (int)(c.c1 - c.c0);
  const int sub = o.G, c16 = o.i16;
  // Row r of the chunk starts at byte r * rsb; the range ends with row L - 1
  // (a row stride is at least one row, so rows >= L fall outside it).  The
  // host keeps 128 row strides within 2^31 bytes.
  const int rsb = (int)(p.m.rs * 2);
  const int flip = (NEG && rsb < 0) ? L - 1 : 0;
  const int span = (NEG && rsb < 0) ? -rsb : rsb;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (bf16 *)p.out + chunk_row_base<REV>(p.m, h, c) + (c.c0 + flip) * p.m.rs, 0, (L - 1) * span + D * 2,
      kRawBufferWord3);
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    const int r0 = 16 * o.qblock(bi) + sub;
    const unsigned rb = Os + kv_off(r0, c16 * 16);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      u32x4 x = lds_ld<u32x4>((rb ^ (it << 4)) + 1024 * it);
      if constexpr (EPI) {
        const bf16x8 o8 = __builtin_bit_cast(bf16x8, x);
        const bf16x8 g8 = __builtin_bit_cast(bf16x8, ep->gr[4 * bi + it]);
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float gate =
              ep->gate ? __builtin_amdgcn_rcpf(1.f + fast_exp2(-(float)g8[e] * kLog2e)) : 1.f;
          y[e] = (float)o8[e] * ep->wt[e] * gate;
        }
        x = __builtin_bit_cast(u32x4, cvt8(y));
      }
      const int r = r0 + 4 * it;
      const int off = (NEG && r >= L) ? (int)0x80000000u : (r - flip) * rsb + c16 * 16;
      __builtin_amdgcn_raw_buffer_store_b128(x, rsrc, off, 0, kCpolNT);
    }
  }
}

// The gate values write_rows<.., EPI> applies to chunk c's rows (rows past
// the chunk's end read its last row: their outputs are never stored).
__device__ __forceinline__ void issue_gate_loads(const FwdArgs &p, int h, const Cursor &c,
                                                 u32x4 (&gr)[8], const OutLane &o) {
  const int Lc = (int)(c.c1 - c.c0);
  const bf16 *base = (const bf16 *)p.gate + p.m.row_base<false>(h, c.j) + c.c0 * p.m.rs + 8 * o.i16;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = 16 * o.qblock(bi) + o.G + 4 * it;
      gr[4 * bi + it] =
          __builtin_nontemporal_load((const u32x4 *)(base + (int64_t)(r < Lc ? r : Lc - 1) * p.m.rs));
    }
}

// RMS normalisation of this lane's two query rows (acc[bi][jt] register r:
// feature 16 jt + 4 G + r; the row's other features sit in the lanes with
// the same i16, lane ^ 16, ^ 32, ^ 48).
__device__ __forceinline__ void rms_rows(f32x4 (&acc)[2][8], float eps) {
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    float ss = 0.f;
#pragma unroll
    for (int jt = 0; jt < 8; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) ss += acc[bi][jt][r] * acc[bi][jt][r];
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float inv = __builtin_amdgcn_rsqf(ss * (1.f / D) + eps);
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) acc[bi][jt] *= inv;
  }
}

// LDS use of the chunk loop.  Chunk n of the walk uses buffer n % 2 (its K
// tile, then its V tile); S^T follows the two buffers.  The tiles arrive by
// direct loads from the state waves: chunk n + 1's K and V tiles go into the
// other buffer during chunk n's state update, one instruction of each per
// update step (by then that buffer's V tile has been read and its K tile's
// staged output rows of chunk n - 1 written back), so the loads stream in
// evenly through the busiest part of the chunk instead of in one burst that
// backs up the CU's memory queue.  After chunk n closes, its K tile holds
// the output waves' staged output rows until they are written back.
//
// Per chunk, two barriers shared by both roles:
//   A (opens the chunk): its K/V tiles and the S^T of the state entering it
//     are in LDS.  Output waves: inter-block term, then intra-block term;
//     state waves: the state update.
//   B (closes it): every read of its K/V tiles and of S^T is done.  Output
//     waves: stage and write back the outputs; state waves: publish the next
//     S^T and wait for the next chunk's tiles.
// The inter-block term thus overlaps the state update instead of waiting
// for it, and both heavy phases sit between A and B.
//
// The intra-block term runs on 16x16x32 MFMA tiles: output wave w owns the
// 16-row query blocks w and 7 - w, so every wave has the same causal work
// (nine 16-key blocks of K Q^T and five 32-key steps of V^T P^T).
//
// Intra-block term of query block bi (rows 16 rb + i16) over the 32-key
// steps kp <= rb / 2: P^T = K Q^T for keys 32 kp + (0..15) (p0) and
// 32 kp + 16 + (0..15) (p1; wholly above the diagonal in the last step of an
// even block, where the mask zeroes it: computing it anyway keeps the step
// free of branches); register r of p0 holds key 32 kp + 4 G + r, of p1 key
// 32 kp + 16 + 4 G + r.  Masked and decayed (lambda^(row - key), zero above
// the diagonal), then O^T += V^T P^T with V read in the same key order.
// Ks, Vs: LDS addresses of the chunk's K and V tiles; kq, vq: this lane's
// tile offsets (see output_loop).
// Masked, decayed scores of one 32-key step as the B operand of V^T P^T:
// p0 holds keys 32 kp + 4 G + r, p1 keys 32 kp + 16 + 4 G + r (r = 0..3) of
// query row `row`; n0 = row - (32 kp + 4 G).  Weight lambda^(row - key),
// zero above the diagonal.
template <bool FAST>
__device__ __forceinline__ bf16x8 decay_mask(const f32x4 &p0, const f32x4 &p1, int n0,
                                             const Decay &dc) {
  const float l2 = dc.l2;
  const int n1 = n0 - 16;
  float pw[8];
  if constexpr (FAST) {
    const float e0 = fast_exp2((float)(n0 - 3) * l2), e1 = fast_exp2((float)(n1 - 3) * l2);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pw[r] = (n0 >= r) ? p0[r] * (e0 * dc.tail[4 + r]) : 0.f;
      pw[4 + r] = (n1 >= r) ? p1[r] * (e1 * dc.tail[4 + r]) : 0.f;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pw[r] = (n0 >= r) ? p0[r] * fast_exp2((float)(n0 - r) * l2) : 0.f;
      pw[4 + r] = (n1 >= r) ? p1[r] * fast_exp2((float)(n1 - r) * l2) : 0.f;
    }
  }
  return cvt8(pw);
}

template <bool FAST, int BI>
__device__ __forceinline__ void intra_block(f32x4 (&acc)[2][8], const u32x4 (&qf)[2][4],
                                            unsigned Ks, unsigned Vs, unsigned kq, unsigned vq,
                                            int i16, int G, int rb, const Decay &dc,
                                            int kp0 = 0) {
  const int row = 16 * rb + i16;
  for (int kp = kp0; kp <= (rb >> 1); ++kp) {
    const unsigned kb = Ks + 32 * kp * KV_ROW + kq;
    f32x4 p0 = {}, p1 = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      p0 = mma16(lds_ld<bf16x8>(kb ^ (ks << 6)), as_bf16x8(qf[BI][ks]), p0);
      p1 = mma16(lds_ld<bf16x8>((kb ^ (ks << 6)) + 16 * KV_ROW), as_bf16x8(qf[BI][ks]), p1);
    }
    const bf16x8 pb = decay_mask<FAST>(p0, p1, row - (32 * kp + 4 * G), dc);
    const unsigned vb = Vs + 32 * kp * KV_ROW + vq;
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      const unsigned va = vb ^ (jt << 5);
      acc[BI][jt] = mma16(tr_read8u(va, va + 16 * KV_ROW), pb, acc[BI][jt]);
    }
  }
}

// Both query blocks of an output wave, w and 7 - w: the key steps of block w
// are the first steps of block 7 - w, so those steps read each K and V
// fragment once for both blocks (two independent product chains per
// fragment); block 7 - w then runs its remaining steps alone.  mid() runs
// between the two parts, once block w's Q^T fragments are spent.
template <bool FAST, typename Mid>
__device__ __forceinline__ void intra_pair(f32x4 (&acc)[2][8], const u32x4 (&qf)[2][4],
                                           unsigned Ks, unsigned Vs, unsigned kq, unsigned vq,
                                           int i16, int G, int w, const Decay &dc,
                                           const Mid &mid) {
  const int row0 = 16 * w + i16, row1 = 16 * (7 - w) + i16;
  for (int kp = 0; kp <= (w >> 1); ++kp) {
    const unsigned kb = Ks + 32 * kp * KV_ROW + kq;
    f32x4 a0 = {}, a1 = {}, b0 = {}, b1 = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 k0 = lds_ld<bf16x8>(kb ^ (ks << 6));
      const bf16x8 k1 = lds_ld<bf16x8>((kb ^ (ks << 6)) + 16 * KV_ROW);
      a0 = mma16(k0, as_bf16x8(qf[0][ks]), a0);
      a1 = mma16(k1, as_bf16x8(qf[0][ks]), a1);
      b0 = mma16(k0, as_bf16x8(qf[1][ks]), b0);
      b1 = mma16(k1, as_bf16x8(qf[1][ks]), b1);
    }
    const int n0 = -(32 * kp + 4 * G);
    const bf16x8 pa = decay_mask<FAST>(a0, a1, row0 + n0, dc);
    const bf16x8 pb = decay_mask<FAST>(b0, b1, row1 + n0, dc);
    const unsigned vb = Vs + 32 * kp * KV_ROW + vq;
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      const unsigned va = vb ^ (jt << 5);
      const bf16x8 vf = tr_read8u(va, va + 16 * KV_ROW);
      acc[0][jt] = mma16(vf, pa, acc[0][jt]);
      acc[1][jt] = mma16(vf, pb, acc[1][jt]);
    }
  }
  mid();
  intra_block<FAST, 1>(acc, qf, Ks, Vs, kq, vq, i16, G, 7 - w, dc, (w >> 1) + 1);
}

// Stages this output wave's accumulators (acc[bi][jt] register r holds
// feature 16 jt + 4 G + r of row 16 qblock(bi) + i16) as bf16 in the
// swizzled tile at LDS address Os: at kv_off(row, 8 G) ^ (jt << 5).
__device__ __forceinline__ void stage_rows(const f32x4 (&acc)[2][8], unsigned Os,
                                           const OutLane &o) {
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    const unsigned sb = Os + kv_off(16 * o.qblock(bi) + o.i16, 8 * o.G);
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      bf16x4 v = {(bf16)acc[bi][jt][0], (bf16)acc[bi][jt][1], (bf16)acc[bi][jt][2],
                  (bf16)acc[bi][jt][3]};
      lds_st<bf16x4>(sb ^ (jt << 5), v);
    }
  }
}

// The chunk loop over segment [cur.c0, b) of head h, output side.  On entry
// qn holds (or is loading) the first chunk's Q^T fragments.
// FAST: the decay weights take the factored powers (see Decay); a template
// parameter so that each chunk step is one basic block the scheduler can
// interleave freely.
// EPI: the gated reading's parts (FwdArgs::flags): SiLU on Q^T as it is
// used, RMS normalisation of the float32 rows, weight and gate at the store
// (the state waves apply the SiLU to the K/V tiles).
template <bool FAST, bool SNAP, bool REV = false, bool EPI = false>
__device__ __forceinline__ void output_loop(const FwdArgs &p, int h, int64_t b, Cursor cur,
                                            u32x4 (&qn)[2][4], char *smem, const Decay &dc,
                                            const Lanes &ln) {
  const SeqMap &m = p.m;
  const int w = ln.w;
  const float l2 = dc.l2;
  const unsigned STs = lds_u32(smem + 2 * LDS_KV);
  f32x4 acc[2][8];
  u32x4 qf[2][4];
  int buf = 0;
  int ci = 0;  // chunk count (phase marks only)
  const bool pm = !SNAP && !REV && !EPI && w == 0;
  Epi ep;
  if constexpr (EPI) {
    // this lane's 8 channels 8 i16 .. of the weight, for the whole walk
    const OutLane o(ln.lane, w);
    const bool wn = (p.flags & GF_NORM) && p.norm_w;
#pragma unroll
    for (int e = 0; e < 8; ++e) ep.wt[e] = wn ? p.norm_w[(int64_t)h * D + 8 * o.i16 + e] : 1.f;
    ep.gate = (p.flags & GF_GATE) != 0;
  }

  while (true) {
    const Cursor nxt = next_chunk<SNAP>(m, cur, b, T);
    const unsigned Ks = lds_u32(smem + buf * LDS_KV), Vs = Ks + LDS_K;
    __syncthreads();  // A: this chunk's K/V and entering S^T are in LDS
    phase_mark(pm, ci, 0, ln.lane);
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qf[bi][ks] = (EPI && (p.flags & GF_SILU_Q)) ? silu8(qn[bi][ks]) : qn[bi][ks];
    {
      const OutLane o(ln.lane, w);
      const int i16 = o.i16, G = o.G;
      // Tile offsets of this lane (see lds_u32): rows 16 n + i16 (K or S^T),
      // granule 4 ks + G (A operand of K Q^T and S^T Q^T): kq ^ (ks << 6);
      // V rows 4 G + (0..3) (+ 16), columns 16 jt .. 16 jt + 15 (transposed
      // reads): vq ^ (jt << 5).
      const unsigned kq = kv_off(i16, 16 * G);
      const unsigned vq = kv_off(4 * G + (i16 >> 2), 8 * (i16 & 3));
      float a_row[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
        a_row[bi] = fast_exp2((float)(16 * o.qblock(bi) + i16 + 1) * l2);

      // The next chunk's Q^T: block 0 now, block 1 once this chunk's block 0
      // fragments are spent (keeps one 16-register set fewer alive).
      if (nxt.valid) issue_q_loads<REV>(p, h, nxt, 0, qn[0], o);
      inter_term(acc, STs + kq, qf, a_row);
      phase_mark(pm, ci, 1, ln.lane);
      intra_pair<FAST>(acc, qf, Ks, Vs, kq, vq, i16, G, w, dc, [&] {
        phase_mark(pm, ci, 2, ln.lane);
        if (nxt.valid) issue_q_loads<REV>(p, h, nxt, 1, qn[1], o);
        if constexpr (EPI) {
          // (the scheduling barrier keeps the gate loads out of the products
          // above, where their registers would be live)
          __builtin_amdgcn_sched_barrier(0);
          if (ep.gate) issue_gate_loads(p, h, cur, ep.gr, o);
        }
      });
      phase_mark(pm, ci, 3, ln.lane);
      if constexpr (EPI) {
        if (p.flags & GF_NORM) rms_rows(acc, p.eps);
      }
    }
    __syncthreads();  // B: this chunk's K/V and S^T reads are done
    phase_mark(pm, ci, 4, ln.lane);
    {
      // Stage the tile in this wave's rows of the chunk's K tile, then write
      // it back as whole rows.
      const OutLane o(ln.lane, w);
      stage_rows(acc, Ks, o);
      write_rows<SNAP, REV, EPI>(p, h, cur, Ks, o, &ep);
    }
    phase_mark(pm, ci++, 5, ln.lane);
    if (!nxt.valid) break;
    cur = nxt;
    buf ^= 1;
  }
}

// The chunk loop, state side.  On entry S holds the state entering the
// segment.  Loads every K/V tile of the walk but the output waves' K tiles
// (see above), updates the state and publishes it as S^T; writes every
// sequence end's final state inside the segment, and the state at every
// snapshot point the segment's chunks end on.
// MID: the output side closes a third barrier in the middle of each chunk
// (the fused dk/dv loop), and the next chunk's tiles go out after it.
// EPI: the gated reading's SiLU on K and/or V (FwdArgs::flags), applied in
// LDS to the rows this wave loaded, once they have landed: the next chunk's
// tiles after this chunk's update (while the output waves finish it).
template <bool SNAP, bool REV = false, bool MID = false, bool EPI = false>
__device__ __forceinline__ void state_loop(const FwdArgs &p, int h, int64_t b, Cursor cur,
                                           f32x16 (&S)[4], char *smem, const Decay &dc,
                                           const Lanes &ln) {
  char *STs = smem + 2 * LDS_KV;
  const SeqMap &m = p.m;
  const int H = m.H;
  const int64_t DD = (int64_t)D * D;
  const int w = ln.w, l32 = ln.l32, g = ln.g, lane = ln.lane;
  const float l2 = dc.l2;
  int buf = 0;
  int ci = 0;  // chunk count (phase marks only)
  const bool pm = !SNAP && !REV && !EPI && !MID && w == 0;
  // Forward views without snapshots: a chunk's row r sits at its first row
  // plus r * rs elements (rs is d or H d), and a whole tile's byte offsets
  // fit 31 bits for any row stride below 2^23 elements.
  constexpr bool PLAIN = !SNAP && !REV;
  const bool plain = PLAIN && m.rs > 0 && m.rs < (int64_t(1) << 23);
  const int rsb = (int)(m.rs * 2);
  // SiLU in place on this wave's rows 32 w .. 32 w + 31 of a K or V tile
  // (elementwise, so the swizzle does not matter).
  const auto silu_rows = [&](char *tile) {
    const unsigned base = lds_u32(tile) + 32 * w * KV_ROW;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned a = base + 16 * (lane + 64 * i);
      lds_st<u32x4>(a, silu8(lds_ld<u32x4>(a)));
    }
  };
  const int silu_k = EPI ? (p.flags & GF_SILU_K) : 0, silu_v = EPI ? (p.flags & GF_SILU_V) : 0;
  dma_tile_rows<REV>(smem, p.k, p, h, cur, w, lane);
  dma_tile_rows<REV>(smem + LDS_K, p.v, p, h, cur, w, lane);
  write_st(STs, S, w, l32, g);
  vm_wait<0>();
  if constexpr (EPI) {
    if (silu_k) silu_rows(smem);
    if (silu_v) silu_rows(smem + LDS_K);
  }

  while (true) {
    const Cursor nxt = next_chunk<SNAP>(m, cur, b, T);
    const int L = (int)(cur.c1 - cur.c0);
    char *Ks = smem + buf * LDS_KV, *Vs = Ks + LDS_K;
    char *Kn = smem + (buf ^ 1) * LDS_KV, *Vn = Kn + LDS_K;
    __syncthreads();  // A: this chunk's K/V and entering S^T are in LDS
    phase_mark(pm, ci, 8, lane);
    // The next chunk's tiles, one K and one V instruction per update step.
    // (The lane id passes through an empty asm statement at each step, so
    // the per-lane address arithmetic is redone there instead of sixteen
    // addresses being hoisted out of the update and held in registers.)
    // A whole chunk of a plain view goes out from uniform row bases with
    // 32-bit lane offsets (dma_quad_whole).
    const bool whole = plain && nxt.valid && (nxt.c1 - nxt.c0) == T;
    const int64_t nrow = whole ? chunk_row_base<REV>(m, h, nxt) + nxt.c0 * m.rs : 0;
    const char *kbn = (const char *)((const bf16 *)p.k + nrow);
    const char *vbn = (const char *)((const bf16 *)p.v + nrow);
    const auto issue_next = [&](int k) {
      if (nxt.valid) {
        int ll = lane;
        asm volatile("" : "+v"(ll));
        if (whole) {
          dma_quad_whole(Kn, kbn, rsb, w, ll, k);
          dma_quad_whole(Vn, vbn, rsb, w, ll, k);
        } else {
          dma_tile_quad<REV>(Kn, p.k, p, h, nxt, w, ll, k);
          dma_tile_quad<REV>(Vn, p.v, p, h, nxt, w, ll, k);
        }
      }
    };
    const bool seq_done = (cur.c1 == cur.seq_end);
    const bool new_piece = nxt.valid && (nxt.c0 >= cur.pend);
    const bool snap_here = SNAP && (cur.c1 == cur.snap);
    if ((nxt.valid && !new_piece) || (seq_done && p.fin) || snap_here) {
      const float gL = fast_exp2((float)L * l2);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) S[nt] *= gL;
      if constexpr (MID)
        state_update(S, Ks, Vs, L, L - 1, l2, dc.fast, dc.tail, w, lane);
      else
        state_update(S, Ks, Vs, L, L - 1, l2, dc.fast, dc.tail, w, lane, issue_next);
      if (seq_done && p.fin) {
        if constexpr (MID) {
          // the backward's dv pass may write lambda times its final state
          // (the walk then starts a new sequence, whose state is loaded)
          if (p.state_scale & 2) {
            const float f = p.decay[h];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) S[nt] *= f;
          }
        }
        store_state(p.fin + ((int64_t)cur.j * H + h) * DD, S, w, l32, g);
      }
      if (snap_here) store_state(p.snaps + (snap_row(m, p.snap_off, cur) * H + h) * DD, S, w, l32, g);
    } else if constexpr (!MID) {
#pragma unroll
      for (int k = 0; k < 8; ++k) issue_next(k);
    }
    phase_mark(pm, ci, 9, lane);
    if constexpr (MID) {
      __syncthreads();  // M: the other buffer's K tile is free again
#pragma unroll
      for (int k = 0; k < 8; ++k) issue_next(k);
    }
    if constexpr (EPI) {
      if (nxt.valid && (silu_k | silu_v)) {
        vm_wait<0>();  // this wave's rows of the next tiles have landed
        if (silu_k) silu_rows(Kn);
        if (silu_v) silu_rows(Vn);
      }
    }
    __syncthreads();  // B: this chunk's K/V and S^T reads are done
    phase_mark(pm, ci, 10, lane);
    if (!nxt.valid) break;
    // (A new piece's state load sits in the same block as the S^T write that
    // consumes it, so no path reaches the next chunk with those loads open.)
    if (new_piece) {
      load_state(S, p.init ? p.init + ((int64_t)nxt.j * H + h) * DD : nullptr, w, l32, g);
      if constexpr (MID) {
        if (p.state_scale & 1) {
          const float f = 1.f / p.decay[h];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) S[nt] *= f;
        }
      }
    }
    write_st(STs, S, w, l32, g);
    phase_mark(pm, ci, 11, lane);
    vm_wait<0>();  // the next chunk's tiles have landed
    phase_mark(pm, ci++, 12, lane);
    cur = nxt;
    buf ^= 1;
  }
}

// Phase C: outputs (and final states) for one (segment, head), from the
// segment's entering state (scan result, initial state or zero).
// SERVE: the general variant: the walk also stores prefix-state snapshots
// (when p.m.snap_iv > 0), takes one segment per sequence (when p.seg_len ==
// 0) and accepts a negative row stride (the time-reversed views of the
// backward pass).  Without it the kernel keeps the plain walk's registers.
// REV (with SERVE): the views may also be time-reversed packed views (the
// backward pass over packed sequences, SeqMap::rev_rs).
template <bool SERVE, bool REV = false, bool EPI = false>
__device__ __forceinline__ void chunk_workgroup(const FwdArgs &p, int bid, char *smem) {
  const Lanes ln;
  const SeqMap &m = p.m;
  const int H = m.H;
  const int s = bid / H, h = bid - (bid / H) * H;
  const Decay dc(p.decay[h]);
  int64_t a, b;
  if (SERVE) {
    segment_bounds(p, s, &a, &b);
  } else {
    a = (int64_t)s * p.seg_len;
    b = (a + p.seg_len < m.total) ? a + p.seg_len : m.total;
  }
  const int64_t DD = (int64_t)D * D;
  const Cursor cur = first_chunk<SERVE>(m, a, b, T);
  if (!cur.valid) {
    // One segment per sequence: an empty sequence keeps its initial state.
    if (SERVE && p.seg_len == 0 && p.fin) {
      float *dst = p.fin + ((int64_t)s * H + h) * DD;
      const float *src = p.init ? p.init + ((int64_t)s * H + h) * DD : nullptr;
      for (int e = threadIdx.x; e < D * D; e += NT) dst[e] = src ? src[e] : 0.f;
    }
    return;
  }
  if (ln.out_wave) {
    u32x4 qn[2][4];
    const OutLane o(ln.lane, ln.w);
    issue_q_loads<REV>(p, h, cur, 0, qn[0], o);
    issue_q_loads<REV>(p, h, cur, 1, qn[1], o);
    if (dc.fast)
      output_loop<true, SERVE, REV, EPI>(p, h, b, cur, qn, smem, dc, ln);
    else
      output_loop<false, SERVE, REV, EPI>(p, h, b, cur, qn, smem, dc, ln);
  } else {
    f32x16 S[4];
    const float *s0 = p.ws ? p.ws + ((int64_t)s * p.r_split * H + h) * DD
                           : (p.init ? p.init + ((int64_t)cur.j * H + h) * DD : nullptr);
    load_state(S, s0, ln.w, ln.l32, ln.g);
    state_loop<SERVE, REV, false, EPI>(p, h, b, cur, S, smem, dc, ln);
  }
}

// EPI: the gated reading's SiLU, normalisation and gate (FwdArgs::flags).
template <bool SERVE, bool EPI = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_chunk_kernel(FwdArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  chunk_workgroup<SERVE, false, EPI>(p, blockIdx.x, smem);
}

// The backward's dv and dk output passes in one workgroup per (segment,
// head).  Both passes walk the same time-reversed chunks with the same tiles:
// the dv pass has keys q and values do (queries k), the dk pass keys do and
// values q (queries v), and the dk pass's state is the transpose of the dv
// pass's (G^T against G, see la_backward.h).  So the state waves run the dv
// pass's walk once (tiles q and do, state G, published as G^T), and the
// output waves compute, per chunk,
//   dv^T = diag(a) (G^T K^T) + do^T ((q K^T) (.) D^T)       queries K = k,
//   dk^T = diag(a) (G V^T)   + q^T ((do V^T) (.) D^T)       queries V = v,
// the second with the tiles' roles swapped and the published G^T read
// transposed.  q and do are read once instead of twice, and the state is
// updated once.
// Per chunk the output side has three barriers: A (opens the chunk), M
// (dv is computed, staged in the other buffer's K tile and written back;
// the state waves then start the next chunk's tiles into that buffer) and
// B (every read of the chunk's tiles and of G^T is done; dk is staged in
// the chunk's K tile and written back).  dk's queries load while dv
// computes, the next chunk's dv queries while dk computes.
template <bool FAST, bool REV>
__device__ __forceinline__ void dkdv_output_loop(const FwdArgs &pv, const FwdArgs &pk, int h,
                                                 int64_t b, Cursor cur, u32x4 (&qn)[2][4],
                                                 char *smem, const Decay &dc, const Lanes &ln) {
  const SeqMap &m = pv.m;
  const int w = ln.w;
  const float l2 = dc.l2;
  const unsigned STs = lds_u32(smem + 2 * LDS_KV);
  f32x4 acc[2][8];
  u32x4 qf[2][4];
  int buf = 0;

  while (true) {
    const Cursor nxt = next_chunk<true>(m, cur, b, T);
    const unsigned Ks = lds_u32(smem + buf * LDS_KV), Vs = Ks + LDS_K;
    const unsigned Xs = lds_u32(smem + (buf ^ 1) * LDS_KV);
    __syncthreads();  // A: this chunk's tiles and entering G^T are in LDS
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[bi][ks] = qn[bi][ks];
    {
      const OutLane o(ln.lane, w);
      const int i16 = o.i16, G = o.G;
      const unsigned kq = kv_off(i16, 16 * G);
      const unsigned vq = kv_off(4 * G + (i16 >> 2), 8 * (i16 & 3));
      float a_row[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
        a_row[bi] = fast_exp2((float)(16 * o.qblock(bi) + i16 + 1) * l2);
      issue_q_loads<REV>(pk, h, cur, 0, qn[0], o);
      inter_term(acc, STs + kq, qf, a_row);
      intra_pair<FAST>(acc, qf, Ks, Vs, kq, vq, i16, G, w, dc,
                       [&] { issue_q_loads<REV>(pk, h, cur, 1, qn[1], o); });
    }
    {
      const OutLane o(ln.lane, w);
      stage_rows(acc, Xs, o);
      write_rows<true, REV>(pv, h, cur, Xs, o);
    }
    __syncthreads();  // M: dv is out of the other buffer
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[bi][ks] = qn[bi][ks];
    {
      const OutLane o(ln.lane, w);
      const int i16 = o.i16, G = o.G;
      const unsigned kq = kv_off(i16, 16 * G);
      const unsigned vq = kv_off(4 * G + (i16 >> 2), 8 * (i16 & 3));
      const unsigned t0 = STs + kv_off(8 * G + (i16 >> 2), 8 * (i16 & 3));
      const unsigned t1 = STs + kv_off(8 * G + 4 + (i16 >> 2), 8 * (i16 & 3));
      float a_row[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
        a_row[bi] = fast_exp2((float)(16 * o.qblock(bi) + i16 + 1) * l2);
      if (nxt.valid) issue_q_loads<REV>(pv, h, nxt, 0, qn[0], o);
      inter_term_tr(acc, t0, t1, qf, a_row);
      intra_pair<FAST>(acc, qf, Vs, Ks, kq, vq, i16, G, w, dc, [&] {
        if (nxt.valid) issue_q_loads<REV>(pv, h, nxt, 1, qn[1], o);
      });
    }
    __syncthreads();  // B: this chunk's tile and G^T reads are done
    {
      const OutLane o(ln.lane, w);
      stage_rows(acc, Ks, o);
      write_rows<true, REV>(pk, h, cur, Ks, o);
    }
    if (!nxt.valid) break;
    cur = nxt;
    buf ^= 1;
  }
}

// One (segment, head) of the fused dv/dk pass: pv is the dv pass (q = k,
// k = q, v = do, out = dv; its entering states, initial state and final
// state), pk supplies the dk pass's queries (q = v) and output (out = dk)
// over the same time-reversed view.
template <bool REV>
__device__ __forceinline__ void dkdv_workgroup(const FwdArgs &pv, const FwdArgs &pk, int bid,
                                               char *smem) {
  const Lanes ln;
  const SeqMap &m = pv.m;
  const int H = m.H;
  const int s = bid / H, h = bid - (bid / H) * H;
  const Decay dc(pv.decay[h]);
  int64_t a, b;
  segment_bounds(pv, s, &a, &b);
  const int64_t DD = (int64_t)D * D;
  const Cursor cur = first_chunk<true>(m, a, b, T);
  // pv.state_scale: the initial state enters as init / lambda, the final
  // state leaves as lambda times the state.
  const float init_f = (pv.state_scale & 1) ? 1.f / pv.decay[h] : 1.f;
  const float fin_f = (pv.state_scale & 2) ? pv.decay[h] : 1.f;
  if (!cur.valid) {
    // One segment per sequence: an empty sequence keeps its initial state.
    if (pv.seg_len == 0 && pv.fin) {
      float *dst = pv.fin + ((int64_t)s * H + h) * DD;
      const float *src = pv.init ? pv.init + ((int64_t)s * H + h) * DD : nullptr;
      for (int e = threadIdx.x; e < D * D; e += NT) dst[e] = src ? fin_f * (init_f * src[e]) : 0.f;
    }
    return;
  }
  if (ln.out_wave) {
    u32x4 qn[2][4];
    const OutLane o(ln.lane, ln.w);
    issue_q_loads<REV>(pv, h, cur, 0, qn[0], o);
    issue_q_loads<REV>(pv, h, cur, 1, qn[1], o);
    if (dc.fast)
      dkdv_output_loop<true, REV>(pv, pk, h, b, cur, qn, smem, dc, ln);
    else
      dkdv_output_loop<false, REV>(pv, pk, h, b, cur, qn, smem, dc, ln);
  } else {
    f32x16 S[4];
    const float *s0 = pv.ws ? pv.ws + ((int64_t)s * pv.r_split * H + h) * DD
                            : (pv.init ? pv.init + ((int64_t)cur.j * H + h) * DD : nullptr);
    load_state(S, s0, ln.w, ln.l32, ln.g);
    if (!pv.ws && (pv.state_scale & 1))  // (the scan's entering states are already scaled)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) S[nt] *= init_f;
    state_loop<true, REV, true>(pv, h, b, cur, S, smem, dc, ln);
  }
}

template <bool REV>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_dkdv_kernel(FwdArgs pv, FwdArgs pk) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  dkdv_workgroup<REV>(pv, pk, blockIdx.x, smem);
}

// Single-pass prefill with the segment scan folded in (MiniMax-01 report,
// section 3.2.2, LASP+: local prefix state, combine with the preceding
// prefix, local outputs -- here between segments of one GPU).  Workgroups
// take segments in ticket order (segment-major, heads fastest); each one
//   1. computes its segment's local state L (K/V streamed from HBM),
//   2. receives the state entering its segment from the workgroup of the
//      previous segment of the same head (a flag and a float32 record in the
//      workspace), and publishes its own end state gamma * S_in + L,
//   3. runs the chunk loop from that entering state; its K/V re-reads come
//      from the Infinity Cache, since segments are short enough for every
//      resident workgroup's K/V to stay there.
// A workgroup only ever waits on a lower ticket, which a running workgroup
// already holds, so the waits cannot deadlock.  A wait that still exceeds
// kSpinLimit polls (a safety net: it would take a stalled GPU) gives up, sets
// *err and continues from a NaN entering state, so that the segment's
// outputs, its end state and every later segment of the head come out NaN:
// never a silently wrong result, and never a hang.
// Ordering: the records are written with agent-scope atomic stores and
// waited for (s_waitcnt) before a workgroup barrier; the flag is then
// published after an agent-scope release fence.  One lane of the waiting
// workgroup polls the flag with relaxed loads; behind the next barrier every
// state wave loads it once more with agent-scope acquire ordering before it
// reads the record.
struct FusedArgs {
  FwdArgs f;         // f.ws: end-state records [nseg][H][D][D]
  unsigned *flags;   // [nseg * H], zero on entry: record published
  unsigned *ticket;  // zero on entry
  unsigned *err;     // set to 1 if a wait timed out
};

constexpr int kSpinLimit = 1 << 18;

__global__ void fused_reset_kernel(unsigned *words, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) words[i] = 0u;
}

// Hand-off records use device-scope (agent) atomic accesses, which are
// coherent across the XCD-private L2 caches; the flag that publishes a
// record is ordered after it by the release fence and the acquire load
// described above (one of each per workgroup).
__device__ __forceinline__ float load_handoff(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_handoff(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// X (local state L on entry) <- the state entering the segment, read from
// `prev` (the previous segment's record when `prev_is_record`, else the
// sequence's initial state, or zero when NULL).  When `publish`, also writes
// gamma * base + L to the record `rec`, with base = the entering state
// (from_prev) or the last piece's own initial state `ini_last`.
// poison: the entering state is NaN (a timed-out wait).
__device__ __forceinline__ void combine_states(f32x16 (&X)[4], const float *prev,
                                               bool prev_is_record, const float *ini_last,
                                               bool from_prev, bool publish, float gam,
                                               float *rec, int u, int l32, int g, bool poison) {
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int off = (32 * u + 8 * q + 4 * g) * D + l32;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const int o = off + mm * D + 32 * nt;
        const float in = poison ? nan
                         : !prev ? 0.f : prev_is_record ? load_handoff(prev + o) : prev[o];
        if (publish) {
          const float base = from_prev ? in : (ini_last ? ini_last[o] : 0.f);
          store_handoff(rec + o, gam * base + X[nt][4 * q + mm]);
        }
        X[nt][4 * q + mm] = in;
      }
  }
}

template <bool SNAP>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_fused_kernel(FusedArgs fa) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  // The ticket passes through the first word of the S^T area, which is not
  // written before the chunk loop starts.
  unsigned *sh_ticket = (unsigned *)(smem + 2 * LDS_KV);
  const FwdArgs &p = fa.f;
  const Lanes ln;
  const SeqMap &m = p.m;
  const int H = m.H;
  if (ln.tid == 0)
    *sh_ticket = __hip_atomic_fetch_add(fa.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const unsigned t = __builtin_amdgcn_readfirstlane(*sh_ticket);
  const int s = (int)(t / (unsigned)H), h = (int)(t - (t / (unsigned)H) * (unsigned)H);
  const Decay dc(p.decay[h]);
  const int64_t a = (int64_t)s * p.seg_len;
  const int64_t b = (a + p.seg_len < m.total) ? a + p.seg_len : m.total;
  const int64_t DD = (int64_t)D * D;
  const Cursor cur = first_chunk<SNAP>(m, a, b, T);
  if (!cur.valid) return;
  char *Ks = smem, *Vs = smem + LDS_K;
  const int jf = cur.j;
  const bool need_in = m.start(jf) < a;   // the segment starts inside a sequence
  const int jl = m.seq_of(b - 1);
  const int64_t ps0 = m.start(jl);
  const int64_t ps = ps0 > a ? ps0 : a;   // start of the segment's last piece
  const bool need_out = m.start(jl + 1) > b;  // that sequence continues after b
  const int64_t kvb = m.row_base<false>(h, jl);

  // Both roles pass the same barriers: two per tile of step 1, one after the
  // wait of step 2, one more after the record stores when publishing, then
  // the chunk loop's.
  if (ln.out_wave) {
    // 1. Stream the last piece's K/V tiles through LDS for the state waves.
    if (need_out) {
      u32x4 tk[8], tv[8];
      int64_t t0 = first_weighted(ps, b, dc.l2, T);
      int Lt = (int)((b - t0) < T ? (b - t0) : T);
      load_tile<256>(tk, (const bf16 *)p.k + kvb + t0 * m.rs, m.rs, Lt, ln.tid);
      load_tile<256>(tv, (const bf16 *)p.v + kvb + t0 * m.rs, m.rs, Lt, ln.tid);
      while (t0 < b) {
        store_tile<256>(Ks, tk, ln.tid);
        store_tile<256>(Vs, tv, ln.tid);
        __syncthreads();
        const int64_t t1 = t0 + T;
        if (t1 < b) {
          Lt = (int)((b - t1) < T ? (b - t1) : T);
          load_tile<256>(tk, (const bf16 *)p.k + kvb + t1 * m.rs, m.rs, Lt, ln.tid);
          load_tile<256>(tv, (const bf16 *)p.v + kvb + t1 * m.rs, m.rs, Lt, ln.tid);
        }
        __syncthreads();
        t0 = t1;
      }
    }
    // 2. The first chunk's Q loads go out while waiting for the entering state.
    u32x4 qn[2][4];
    const OutLane o(ln.lane, ln.w);
    issue_q_loads(p, h, cur, 0, qn[0], o);
    issue_q_loads(p, h, cur, 1, qn[1], o);
    if (need_in && ln.tid == 0) {
      const unsigned *fl = fa.flags + (size_t)(s - 1) * H + h;
      int it = 0;
      while (__hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        if (++it > kSpinLimit) {
          __hip_atomic_store(fa.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();  // the state waves' record loads are issued after the flag was seen
    if (need_out) {
      __syncthreads();  // the state waves' record stores have completed
      if (ln.tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_store(fa.flags + (size_t)s * H + h, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // 3. Outputs from the entering state.
    if (dc.fast)
      output_loop<true, SNAP>(p, h, b, cur, qn, smem, dc, ln);
    else
      output_loop<false, SNAP>(p, h, b, cur, qn, smem, dc, ln);
  } else {
    // 1. L = sum over the last piece of lambda^(b-1-c) k_c^T v_c.
    f32x16 S[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[nt] = (f32x16){};
    if (need_out) {
      int64_t t0 = first_weighted(ps, b, dc.l2, T);
      while (t0 < b) {
        const int Lc = (int)((b - t0) < T ? (b - t0) : T);
        __syncthreads();
        state_update(S, Ks, Vs, Lc, (int)(b - 1 - t0), dc.l2, dc.fast, dc.tail, ln.w, ln.lane);
        __syncthreads();
        t0 += T;
      }
    }
    // 2. S <- the entering state, and the end state is published.
    __syncthreads();  // the flag of the previous segment has been seen
    const float *prev = need_in ? p.ws + ((int64_t)(s - 1) * H + h) * DD
                                : (p.init ? p.init + ((int64_t)jf * H + h) * DD : nullptr);
    const float *ini_last = p.init ? p.init + ((int64_t)jl * H + h) * DD : nullptr;
    const float gam = fast_exp2((float)(b - ps) * dc.l2);
    // The flag, read again with acquire ordering, makes the record visible;
    // still unset, the wait above timed out and the entering state is poisoned.
    const bool poisoned =
        need_in && __builtin_amdgcn_readfirstlane(__hip_atomic_load(
                       fa.flags + (size_t)(s - 1) * H + h, __ATOMIC_ACQUIRE,
                       __HIP_MEMORY_SCOPE_AGENT)) == 0u;
    combine_states(S, prev, need_in, ini_last, ps == a, need_out, gam,
                   p.ws + ((int64_t)s * H + h) * DD, ln.w, ln.l32, ln.g, poisoned);
    if (need_out) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's record stores have completed
      __syncthreads();
    }
    // 3. Outputs from the entering state.
    state_loop<SNAP>(p, h, b, cur, S, smem, dc, ln);
  }
}

// The head of rank k when heads are ordered by decreasing decay (ties by
// index), for H <= NT_LOCAL.  Ranks compare the decays' bit patterns, a
// strict order for any values, so every head has exactly one rank.  Called
// by every thread of the workgroup; kept out of line so that the caller's
// register allocation is that of its own loop.
__device__ __attribute__((noinline)) int head_by_decay_rank(const float *decay, int H, int k) {
  __shared__ unsigned lam_bits[NT_LOCAL];
  __shared__ int ranked;
  const int tid = threadIdx.x;
  if (tid < H) lam_bits[tid] = __float_as_uint(decay[tid]);
  if (tid == 0) ranked = k;
  __syncthreads();
  if (tid < H) {
    const unsigned x = lam_bits[tid];
    int rank = 0;
    for (int j = 0; j < H; ++j) {
      const unsigned y = lam_bits[j];
      rank += (y > x || (y == x && j < tid)) ? 1 : 0;
    }
    if (rank == k) ranked = tid;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(ranked);
}

// Phase A: the local state of each segment's last piece, from zero:
//   L_s = sum_{c in [ps, b)} lambda^(b-1-c) k_c^T v_c, one decayed MFMA sum.
// Chunks before first_weighted(ps, b) carry exactly zero weight and are left
// out; the weighted part is cut into up to p.r_split sub-ranges [x0, x1) of
// whole 64-token chunks (piece_plan: fewer for a head whose weighted part is
// short, so that no workgroup walks much more than a piece of a slowly
// decaying head); one workgroup computes each partial state
//   P_r = sum_{c in [x0, x1)} lambda^(x1-1-c) k_c^T v_c
// into slot (s, r), and the scan forms L_s = sum_r lambda^(b - x1_r) P_r.
// Small workgroups (4 waves, 32 KB of LDS, two chunks in flight) several to
// a CU hide one another's load and arithmetic latency.
// Grid: (nseg - 1) * r_split * H workgroups (the last segment hands no
// state on), piece-major from the last piece down; within a piece index
// heads fastest, segments in reverse (the K/V read last are the first
// segments', which the output pass reads first: Infinity Cache), except the
// first pieces, which go slowest head first (below); items spread over the
// XCDs by xcd_spread (a head's pieces are long or short with its decay).
// (Ordering the whole grid by decreasing decay, before the piece-major
// order, measured slower.)
// Wave u owns state rows 32u..32u+31.
// CH: channel-wise decay (p.chdecay): row c's K values are scaled by their
// channel's alpha_i^(x1-1-c) on the way into LDS and the update runs with
// unit weights; chunks are skipped with the slowest channel's decay.
// SILU: the gated path's SiLU on K and V (p.flags) is applied as they are
// staged.
template <bool CH = false, bool SILU = false>
__global__ __launch_bounds__(NT_LOCAL) __attribute__((amdgpu_waves_per_eu(2, 4)))
void local_state_kernel(FwdArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * C_LOCAL * KV_ROW];
  char *Ks = smem, *Vs = smem + C_LOCAL * KV_ROW;
  const int tid = threadIdx.x, lane = tid & 63, u = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const SeqMap &m = p.m;
  const int H = m.H, R = p.r_split;
  // Items piece-major from the last piece down, heads fastest (spread over
  // the XCDs): the slowly decaying heads' extra pieces, all of full length,
  // go out first, and every head's first piece -- among them the short
  // single pieces of fast heads -- last, where they fill the gaps of the
  // final round instead of starting a round of long pieces of their own.
  // Among the first pieces the slowest heads go first (longest first), so
  // that the shortest are the very last: 3-7% off the pass at 16-64 heads of
  // 131K-512K tokens, level at 8 heads x 1M tokens and at the 64-head
  // 32K-token layer.
  const int item = xcd_spread((int)blockIdx.x, (int)gridDim.x);
  const int per_r = (p.nseg - 1) * H;
  const int rr = item / per_r, rem = item - rr * per_r;
  const int r = R - 1 - rr;
  int idx = rem / H, h = rem - idx * H;
  if (!CH && r == 0 && H <= NT_LOCAL) {
    // The first pieces, slowest heads first (segments fastest): a slowly
    // decaying head's first piece is as long as its others, a fast head's
    // single piece short.  (The channel-wise pass would need every channel's
    // decay to rank a head; it keeps the plain order.)
    const int k = rem / (p.nseg - 1);
    idx = rem - k * (p.nseg - 1);
    h = head_by_decay_rank(p.decay, H, k);
  }
  const int s = p.nseg - 2 - idx;
  float l2max = 0.f, l2f[8];  // channel-wise: slowest channel, and this thread's 8 channels
  if constexpr (CH) {
    const float *al = p.chdecay + (int64_t)h * D;
    l2max = -__builtin_huge_valf();
    for (int i = 0; i < D; ++i) l2max = fmaxf(l2max, log2f(al[i]));
    l2max = uniform(l2max);
#pragma unroll
    for (int e = 0; e < 8; ++e) l2f[e] = log2f(al[8 * (tid & 15) + e]);
  }
  const float l2 = CH ? 0.f : uniform(log2f(p.decay[h]));  // CH: unit weights in the update
  const bool fast = l2 > kFastLog2;
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
  const Pieces P = piece_plan(ps, b, CH ? l2max : l2, C_LOCAL, R);
  if (r >= (1 << P.lg)) return;
  int64_t r0, x1;
  piece_range(P, b, C_LOCAL, r, &r0, &x1);
  if (r0 >= x1) return;
  float tail[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) tail[i] = uniform(fast_exp2((float)(7 - i) * l2));

  f32x16 S[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) S[nt] = (f32x16){};
  // Two chunks in flight: while chunk t is in LDS and being summed, chunks
  // t + 1 and t + 2 are loading into two register sets.  Loads past the
  // piece's end re-read its last chunk (still in L2; the data go unused), so
  // every load is unconditional and the compiler's memory waits stay exact.
  constexpr int PER = C_LOCAL * 16 / NT_LOCAL;
  u32x4 pk[2][PER], pv[2][PER];
  const int64_t last = r0 + (x1 - 1 - r0) / C_LOCAL * C_LOCAL;  // start of the last chunk
  const bf16 *kb = (const bf16 *)p.k + base, *vb = (const bf16 *)p.v + base;
  auto issue = [&](auto slot_c, int64_t t) {
    constexpr int sl = decltype(slot_c)::value;
    const int64_t tt = t < last ? t : last;
    const int Lt = (int)((x1 - tt) < C_LOCAL ? (x1 - tt) : C_LOCAL);
    load_tile<NT_LOCAL, C_LOCAL>(pk[sl], kb + tt * m.rs, m.rs, Lt, tid);
    load_tile<NT_LOCAL, C_LOCAL>(pv[sl], vb + tt * m.rs, m.rs, Lt, tid);
  };
  // Sums the chunk at t0 held in register set sl, then reloads that set with
  // the chunk two ahead.
  int ci = 0;  // chunk count (phase marks only)
  const bool pm = !CH && !SILU;
  auto step = [&](auto slot_c, int64_t t0) {
    constexpr int sl = decltype(slot_c)::value;
    phase_mark_local(pm, ci, 0, tid);
    if constexpr (CH) {
      // K[c][i] alpha_i^(x1-1-c) for the thread's rows c and channels i
#pragma unroll
      for (int it = 0; it < PER; ++it) {
        const int row = (it * NT_LOCAL + tid) >> 4;
        const float n = (float)(x1 - 1 - (t0 + row));
        const bf16x8 kv = __builtin_bit_cast(bf16x8, pk[sl][it]);
        float ks[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ks[e] = (float)kv[e] * fast_exp2(n * l2f[e]);
        pk[sl][it] = __builtin_bit_cast(u32x4, cvt8(ks));
      }
    }
    if constexpr (SILU) {
      if (p.flags & GF_SILU_K)
#pragma unroll
        for (int it = 0; it < PER; ++it) pk[sl][it] = silu8(pk[sl][it]);
      if (p.flags & GF_SILU_V)
#pragma unroll
        for (int it = 0; it < PER; ++it) pv[sl][it] = silu8(pv[sl][it]);
    }
    store_tile<NT_LOCAL, C_LOCAL>(Ks, pk[sl], tid);
    store_tile<NT_LOCAL, C_LOCAL>(Vs, pv[sl], tid);
    __syncthreads();
    phase_mark_local(pm, ci, 1, tid);
    issue(slot_c, t0 + 2 * C_LOCAL);
    const int Lc = (int)((x1 - t0) < C_LOCAL ? (x1 - t0) : C_LOCAL);
    // weight of chunk row c: lambda^(x1 - 1 - (t0 + c)); the pipelined update
    // (LDS reads a step ahead) fits the two-waves-per-SIMD register budget
    state_update<C_LOCAL / 16, true>(S, Ks, Vs, Lc, (int)(x1 - 1 - t0), l2, fast, tail, u, lane);
    phase_mark_local(pm, ci, 2, tid);
    __syncthreads();
    phase_mark_local(pm, ci++, 3, tid);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // (No branch in the loop body and the two sets issued in order: either
  // would make the compiler wait for every load at the top of the loop.)
  issue(S0{}, r0);
  __builtin_amdgcn_sched_barrier(0);
  issue(S1{}, r0 + C_LOCAL);
  int64_t t0 = r0;
  for (; t0 + C_LOCAL < x1; t0 += 2 * C_LOCAL) {
    step(S0{}, t0);
    step(S1{}, t0 + C_LOCAL);
  }
  if (t0 < x1) step(S0{}, t0);
  // The last loads (past the piece's end) are waited for before the stores
  // below are issued; they read memory the piece already read.
  store_state(p.ws + (((int64_t)s * R + r) * H + h) * (int64_t)D * D, S, u, l32, g);
}

}  // namespace mfma
}  // namespace la
