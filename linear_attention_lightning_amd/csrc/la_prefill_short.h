// bf16 prefill on gfx950 MFMA with short chunks (32 or 64 tokens), d = 128.
//
// The MiniMax-01 report pads its inputs to 32, 64, 128 or 256 tokens by
// length (section 3.3.3, multi-level padding), so that short inputs do not
// pay for a long block.  Here nothing is padded; the block length chooses
// the chunk the kernel walks: this kernel runs 32- or 64-token chunks with a
// small LDS footprint (two tiles and S^T: 56 or 80 KB, two workgroups per
// CU), where the 128-token kernel takes a whole CU per workgroup.  The
// arithmetic per chunk of L rows is the 128-token kernel's (section 2.2.1):
//     O^T = diag(a) (S^T Q^T) + V^T ((K Q^T) (.) D^T),   a_r = lambda^(r+1)
//     S   = lambda^L S + (diag(b) K)^T V,                b_c = lambda^(L-1-c)
// on the same MFMA fragments (16x16x32 for the outputs, 32x32x16 for the
// state), but one workgroup of 4 waves does both in turn: wave w owns query
// rows 16w..16w+15 of a 64-token chunk (a 32-token chunk: rows 16(w&1).. and
// features 64(w>>1)..) and state rows 32w..32w+31.  K and V come through
// registers one chunk ahead, Q likewise; outputs are staged in LDS and
// written back as whole rows at the start of the next chunk, behind its
// first barrier.
#pragma once

#include "la_prefill_mfma.h"

namespace la {
namespace mfma {

constexpr int NT_S = 256;  // threads per workgroup of the short-chunk kernel (4 waves)

template <int TS>
struct ShortLds {
  static constexpr int TILE = TS * KV_ROW;  // one TS x 128 bf16 tile, swizzled rows
  static constexpr int K = 0, V = TILE, O = 2 * TILE, ST = 3 * TILE;
  static constexpr int BYTES = 3 * TILE + LDS_ST;
};

// K and V rows of chunk c into registers (tile rows (it * 256 + t) / 16,
// granule t % 16); rows past the chunk's end repeat its last row.
template <int TS>
__device__ __forceinline__ void short_load_kv(u32x4 (&kr)[TS / 16], u32x4 (&vr)[TS / 16],
                                              const FwdArgs &p, int h, const Cursor &c, int t) {
  const int Lc = (int)(c.c1 - c.c0);
  const int64_t base = p.m.row_base<false>(h, c.j) + c.c0 * p.m.rs;
  load_tile<NT_S, TS>(kr, (const bf16 *)p.k + base, p.m.rs, Lc, t);
  load_tile<NT_S, TS>(vr, (const bf16 *)p.v + base, p.m.rs, Lc, t);
}

// Q^T fragments of chunk row `row` (B operand of the 16x16x32 products:
// q[ks] holds features 32 ks + 8 G .. + 7), non-temporal.
__device__ __forceinline__ void short_load_q(u32x4 (&q)[4], const FwdArgs &p, int h,
                                             const Cursor &c, int row, int G) {
  const int Lc = (int)(c.c1 - c.c0);
  const bf16 *qrow = (const bf16 *)p.q + p.m.row_base<false>(h, c.j) +
                     (c.c0 + (row < Lc ? row : Lc - 1)) * p.m.rs + 8 * G;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    q[ks] = __builtin_nontemporal_load((const u32x4 *)(qrow + 32 * ks));
}

template <int TS>
__global__ __launch_bounds__(NT_S) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_short_kernel(FwdArgs p) {
  static_assert(TS == 32 || TS == 64, "chunk of 32 or 64 tokens");
  using LY = ShortLds<TS>;
  constexpr int PT = TS / 16;              // 16-byte pieces per thread of one tile
  constexpr int NJ = TS == 64 ? 8 : 4;     // 16-feature tiles of a wave's output
  __shared__ __attribute__((aligned(1024))) char smem[LY::BYTES];
  char *Ks = smem + LY::K, *Vs = smem + LY::V, *STs = smem + LY::ST;
  const unsigned Ku = lds_u32(Ks), Vu = lds_u32(Vs), Ou = lds_u32(smem + LY::O);
  const unsigned STu = lds_u32(STs);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const SeqMap &m = p.m;
  const int H = m.H;
  const int s = blockIdx.x / H, h = blockIdx.x - s * H;
  const Decay dc(p.decay[h]);
  const float l2 = dc.l2;
  const int64_t DD = (int64_t)D * D;
  int64_t a, b;
  segment_bounds(p, s, &a, &b);
  Cursor cur = first_chunk<false>(m, a, b, TS);
  if (!cur.valid) {
    // One segment per sequence: an empty sequence keeps its initial state.
    if (p.seg_len == 0 && p.fin) {
      float *dst = p.fin + ((int64_t)s * H + h) * DD;
      const float *src = p.init ? p.init + ((int64_t)s * H + h) * DD : nullptr;
      for (int e = tid; e < D * D; e += NT_S) dst[e] = src ? src[e] : 0.f;
    }
    return;
  }
  const int qb = TS == 64 ? w : (w & 1);   // this wave's 16-row query block
  const int j0 = TS == 64 ? 0 : 4 * (w >> 1);
  const int row0 = 16 * qb + (lane & 15);  // this lane's query row in a chunk

  // Entering state (scan result, initial state or zero), S^T, and the first
  // chunk's tiles and Q.
  f32x16 S[4];
  load_state(S, p.ws ? p.ws + ((int64_t)s * p.r_split * H + h) * DD
                     : (p.init ? p.init + ((int64_t)cur.j * H + h) * DD : nullptr),
             w, l32, g);
  u32x4 kr[PT], vr[PT], qf[4];
  short_load_kv<TS>(kr, vr, p, h, cur, tid);
  short_load_q(qf, p, h, cur, row0, lane >> 4);
  store_tile<NT_S, TS>(Ks, kr, tid);
  store_tile<NT_S, TS>(Vs, vr, tid);
  write_st(STs, S, w, l32, g);

  // Writes the staged outputs of chunk c (rows (it * 256 + t) / 16, granule
  // t % 16) as whole rows, through a buffer whose range ends with the chunk's
  // last row (stores to later rows are dropped).
  auto write_back = [&](const Cursor &c) {
    const int L = (int)(c.c1 - c.c0);
    const int rsb = (int)(m.rs * 2);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (bf16 *)p.out + m.row_base<false>(h, c.j) + c.c0 * m.rs, 0, (L - 1) * rsb + D * 2,
        kRawBufferWord3);
    const int c16 = tid & 15;
#pragma unroll
    for (int it = 0; it < PT; ++it) {
      const int r = (it * NT_S + tid) >> 4;
      const u32x4 x = lds_ld<u32x4>(Ou + kv_off(r, 16 * c16));
      __builtin_amdgcn_raw_buffer_store_b128(x, rsrc, r * rsb + 16 * c16, 0, kCpolNT);
    }
  };

  Cursor prev = cur;
  bool staged = false;
  while (true) {
    const Cursor nxt = next_chunk<false>(m, cur, b, TS);
    const Cursor ld = nxt.valid ? nxt : cur;  // loads past the last chunk re-read it
    const int L = (int)(cur.c1 - cur.c0);
    // Lane coordinates re-derived in every chunk from a lane id the compiler
    // cannot see through: otherwise it hoists every fragment address out of
    // the loop and spills.
    int lid = lane;
    asm volatile("" : "+v"(lid));
    const int i16 = lid & 15, G = lid >> 4;
    const int row = 16 * qb + i16;
    const unsigned kq = kv_off(i16, 16 * G);
    const unsigned vq = kv_off(4 * G + (i16 >> 2), 8 * (i16 & 3));
    __syncthreads();  // A: tiles, S^T of this chunk and the previous chunk's staging
    if (staged) write_back(prev);
    u32x4 qn[4];
    short_load_kv<TS>(kr, vr, p, h, ld, tid);
    short_load_q(qn, p, h, ld, row, G);
    // State update of this wave's rows 32 w .. 32 w + 31 first: the outputs
    // read the entering state from S^T in LDS, so the accumulators below need
    // not live through the update.
    const bool seq_done = (cur.c1 == cur.seq_end);
    const bool new_piece = nxt.valid && (nxt.c0 >= cur.pend);
    if ((nxt.valid && !new_piece) || (seq_done && p.fin)) {
      const float gL = fast_exp2((float)L * l2);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) S[nt] *= gL;
      state_update<TS / 16, true>(S, Ks, Vs, L, L - 1, l2, dc.fast, dc.tail, w, lid);
      if (seq_done && p.fin) store_state(p.fin + ((int64_t)cur.j * H + h) * DD, S, w, l32, g);
    }
    // Outputs of query rows 16 qb + (0..15), features 16 (j0 + j) + 4 G + r.
    bf16x8 qv[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qv[ks] = as_bf16x8(qf[ks]);
    f32x4 acc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      acc[j] = (f32x4){};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc[j] = mma16(lds_ld<bf16x8>(((STu + kq) ^ (ks << 6)) + 4096 * (j0 + j)), qv[ks], acc[j]);
    }
    {
      const float a_row = fast_exp2((float)(row + 1) * l2);
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] *= a_row;
    }
    for (int kp = 0; kp <= (qb >> 1); ++kp) {
      const unsigned kb = Ku + 32 * kp * KV_ROW + kq;
      f32x4 p0 = {}, p1 = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        p0 = mma16(lds_ld<bf16x8>(kb ^ (ks << 6)), qv[ks], p0);
        p1 = mma16(lds_ld<bf16x8>((kb ^ (ks << 6)) + 16 * KV_ROW), qv[ks], p1);
      }
      // register r of p0 holds key 32 kp + 4 G + r, of p1 key 32 kp + 16 + 4 G + r
      const int n0 = row - (32 * kp + 4 * G), n1 = n0 - 16;
      float pw[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pw[r] = (n0 >= r) ? p0[r] * fast_exp2((float)(n0 - r) * l2) : 0.f;
        pw[4 + r] = (n1 >= r) ? p1[r] * fast_exp2((float)(n1 - r) * l2) : 0.f;
      }
      const bf16x8 pb = cvt8(pw);
      const unsigned vb = Vu + 32 * kp * KV_ROW + vq;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const unsigned va = vb ^ ((j0 + j) << 5);
        acc[j] = mma16(tr_read8u(va, va + 16 * KV_ROW), pb, acc[j]);
      }
    }
    __syncthreads();  // B: every read of this chunk's tiles, of S^T and of the staging is done
    // Stage the outputs (acc[j] register r: feature 16 (j0 + j) + 4 G + r of row `row`).
    {
      const unsigned sb = Ou + kv_off(row, 8 * G);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bf16x4 v4 = {(bf16)acc[j][0], (bf16)acc[j][1], (bf16)acc[j][2], (bf16)acc[j][3]};
        lds_st<bf16x4>(sb ^ ((j0 + j) << 5), v4);
      }
    }
    prev = cur;
    staged = true;
    if (!nxt.valid) break;
    if (new_piece)
      load_state(S, p.init ? p.init + ((int64_t)nxt.j * H + h) * DD : nullptr, w, l32, g);
    write_st(STs, S, w, l32, g);
    store_tile<NT_S, TS>(Ks, kr, tid);
    store_tile<NT_S, TS>(Vs, vr, tid);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = qn[ks];
    cur = nxt;
  }
  __syncthreads();  // the last chunk's staging is complete
  write_back(prev);
}

}  // namespace mfma
}  // namespace la
