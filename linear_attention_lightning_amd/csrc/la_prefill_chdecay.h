// Output pass of the channel-wise decay variant on MFMA (bf16, d = 128).
//
// Head h has one decay alpha_i per key channel i (K3 reading notes,
// "gated DeltaNet": channel-wise decay; here without the delta rule):
//   S_t[i][j] = alpha_i S_{t-1}[i][j] + k_t[i] v_t[j],   o_t = q_t S_t.
// Blockwise over chunks of TC tokens, with q the query row and c the key row
// inside a chunk of L tokens:
//   O = (Q (.) alpha^(q+1)) S + P V,   P[q][c] = sum_i Q[q][i] K[c][i] alpha_i^(q-c)  (c <= q)
//   S <- diag(alpha^L) S + (K (.) alpha^(L-1-c))^T V.
// The decay inside P depends on the contracted channel, so P is not a plain
// product of Q and K.  It becomes one by writing decay as an absolute
// position around a pivot (the K3 notes' trick of scaling Q by a decay and K
// by its inverse): alpha_i^(q-c) = alpha_i^(q-32) alpha_i^(32-c), so with
//   Q~ = Q (.) alpha^(q-32),   K~ = K (.) alpha^(32-c)
// P = (Q~ K~^T) masked to c <= q, and the state update reuses K~:
// K (.) alpha^(L-1-c) = K~ (.) alpha^(L-33), one factor per channel.  The
// pivot in the middle of a 64-token chunk keeps every factor within
// alpha^(+-32) (the notes bound the window so that the factors stay inside
// the BF16 range): heads whose smallest alpha is at least 1/8 (factors below
// 2^96) run here, the others on the vector-ALU kernel (kChMinLog2).
//
// Workgroup = (segment, head), 8 waves as in the scalar kernel: output waves
// 0-3 each own query rows 16w..16w+15 of a chunk; state waves 4-7 own state
// rows 32u..32u+31, load K and V two chunks ahead through registers (scaling
// K on the way into LDS) while they update the state, and publish S^T; the
// output waves load Q two chunks ahead likewise.
#pragma once

#include "la_prefill_mfma.h"

namespace la {
namespace mfma {

constexpr int TC = 64;        // tokens per chunk of the channel-wise kernel
constexpr int CH_PIVOT = 32;  // pivot row of the decay factorisation
constexpr int LDS_CH_K = TC * KV_ROW;  // one 64 x 128 bf16 tile (16 KB)
// K~ and V tiles, the output staging tile, S^T, log2 alpha of the head's
// channels.
constexpr int LDS_CH = 3 * LDS_CH_K + LDS_ST + D * 4;

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// State-wave thread ts (0..255): granule c16 = ts % 16 (features 8 c16 ..
// 8 c16 + 7) of rows ts / 16 + 16 it, it = 0..3, of a chunk's K and V.
struct ChTiles {
  u32x4 k[4], v[4];
};

__device__ __forceinline__ void ch_load_tiles(ChTiles &t, const FwdArgs &p, int h,
                                              const Cursor &c, int ts) {
  const int Lc = (int)(c.c1 - c.c0);
  const int64_t base = p.m.row_base<false>(h, c.j) + c.c0 * p.m.rs;
  const bf16 *kb = (const bf16 *)p.k + base, *vb = (const bf16 *)p.v + base;
  const int c16 = ts & 15;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = (ts >> 4) + 16 * it;
    const int rr = row < Lc ? row : Lc - 1;  // rows past the chunk re-read its last row
    t.k[it] = __builtin_nontemporal_load((const u32x4 *)(kb + (int64_t)rr * p.m.rs + 8 * c16));
    t.v[it] = __builtin_nontemporal_load((const u32x4 *)(vb + (int64_t)rr * p.m.rs + 8 * c16));
  }
}

// K~ = K (.) alpha^(32 - row) and V into the swizzled LDS tiles; rows >= L
// are stored as zeros, so they add nothing to any product.  kf[it][e]:
// alpha^(32 - row) of this thread's row (ts >> 4) + 16 it and channel e of
// its 8 channels, the same for every chunk (see ch_tile_factors).
__device__ __forceinline__ void ch_store_tiles(char *Ks, char *Vs, const ChTiles &t, int L,
                                               const float (&kf)[4][8], int ts) {
  const int c16 = ts & 15;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = (ts >> 4) + 16 * it;
    const bool live = row < L;
    const bf16x8 kv = __builtin_bit_cast(bf16x8, t.k[it]);
    float ks[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ks[e] = live ? (float)kv[e] * kf[it][e] : 0.f;
    *(bf16x8 *)(Ks + kv_off(row, 16 * c16)) = cvt8(ks);
    *(u32x4 *)(Vs + kv_off(row, 16 * c16)) = live ? t.v[it] : (u32x4){0u, 0u, 0u, 0u};
  }
}

// The factors of ch_store_tiles: alpha_e^(32 - row) for this thread's rows
// (ts >> 4) + 16 it and channels (l2f: their log2 alpha).
__device__ __forceinline__ void ch_tile_factors(float (&kf)[4][8], const float (&l2f)[8], int ts) {
#pragma unroll
  for (int it = 0; it < 4; ++it)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      kf[it][e] = fast_exp2((float)(CH_PIVOT - ((ts >> 4) + 16 * it)) * l2f[e]);
}

// S += (f K~)^T V over the chunk's TC rows, for state rows 32u..32u+31; f is
// this lane's channel factor (A-operand row 32u + l32).
__device__ __forceinline__ void ch_state_update(f32x16 (&S)[4], const char *Ks, const char *Vs,
                                                float f, int u, int lane) {
  const int g = lane >> 5, G16 = lane >> 4, i16 = lane & 15;
  const int ko0 = tr_off(8 * g, u, G16, i16), ko1 = tr_off(8 * g + 4, u, G16, i16);
  int vo0[4], vo1[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    vo0[nt] = tr_off(8 * g, nt, G16, i16);
    vo1[nt] = tr_off(8 * g + 4, nt, G16, i16);
  }
#pragma unroll
  for (int ks = 0; ks < TC / 16; ++ks) {
    const bf16x8 kf = tr_read8(Ks + 16 * ks * KV_ROW, ko0, ko1);
    float wv[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) wv[s] = (float)kf[s] * f;
    const bf16x8 a = cvt8(wv);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      S[nt] = mma(a, tr_read8(Vs + 16 * ks * KV_ROW, vo0[nt], vo1[nt]), S[nt]);
  }
}

// This output wave's Q^T fragments (B operand of the 16x16x32 products):
// q[ks] holds features 32 ks + 8 G .. + 7 of chunk row 16 w + i16.
__device__ __forceinline__ void ch_issue_q(u32x4 (&q)[4], const FwdArgs &p, int h,
                                           const Cursor &c, int w, int i16, int G) {
  const int Lc = (int)(c.c1 - c.c0);
  const int row = 16 * w + i16;
  const bf16 *qrow = (const bf16 *)p.q + p.m.row_base<false>(h, c.j) +
                     (c.c0 + (row < Lc ? row : Lc - 1)) * p.m.rs + 8 * G;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    q[ks] = __builtin_nontemporal_load((const u32x4 *)(qrow + 32 * ks));
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void chdecay_chunk_kernel(FwdArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS_CH];
  char *Ks = smem, *Vs = smem + LDS_CH_K, *Os = smem + 2 * LDS_CH_K, *STs = smem + 3 * LDS_CH_K;
  float *l2a = (float *)(smem + 3 * LDS_CH_K + LDS_ST);
  const Lanes ln;
  const SeqMap &m = p.m;
  const int H = m.H;
  const int s = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int64_t a = (int64_t)s * p.seg_len;
  const int64_t b = (a + p.seg_len < m.total) ? a + p.seg_len : m.total;
  const int64_t DD = (int64_t)D * D;
  const float *alpha = p.chdecay + (int64_t)h * D;
  // A head with a decay below 2^kChMinLog2 is the vector-ALU kernel's.
  if (p.ch_split == 1 && ch_small_head(alpha, D)) return;
  Cursor cur = first_chunk<false>(m, a, b, TC);
  if (!cur.valid) return;
  if (ln.tid < D) l2a[ln.tid] = log2f(alpha[ln.tid]);  // read after the first barrier

  if (ln.out_wave) {
    const int w = ln.w, i16 = ln.i16, G = ln.G16;
    const int row = 16 * w + i16;  // this lane's query row inside a chunk
    const unsigned kq = kv_off(i16, 16 * G);
    const unsigned vq = kv_off(4 * G + (i16 >> 2), 8 * (i16 & 3));
    const unsigned st = lds_u32(STs) + kq;
    const unsigned kbase = lds_u32(Ks), vbase = lds_u32(Vs);
    // Q two chunks ahead in two register sets; loads past the segment's
    // last chunk re-read it (never used), so every load is unconditional.
    u32x4 qn[2][4];
    Cursor nxt = next_chunk<false>(m, cur, b, TC);
    ch_issue_q(qn[0], p, h, cur, w, i16, G);
    ch_issue_q(qn[1], p, h, nxt.valid ? nxt : cur, w, i16, G);
    // The two scalings of this lane's Q features (32 ks + 8 G + e of query
    // row `row`): alpha^(row+1) for the inter term, alpha^(row-32) for the
    // intra term.  The same for every chunk, so taken once (after the first
    // barrier, once l2a is in LDS) instead of 64 exponentials per chunk.
    float fi[4][8], ft[4][8];
    bool have_f = false;
    // One chunk: Q of `c` is in set sl; reloads set sl with chunk c + 2.
    // Returns false after the segment's last chunk.
    auto step = [&](auto slot_c, const Cursor &c, const Cursor &n1) -> bool {
      constexpr int sl = decltype(slot_c)::value;
      const Cursor n2 = n1.valid ? next_chunk<false>(m, n1, b, TC) : n1;
      __syncthreads();  // A: K~, V and S^T of this chunk are in LDS
      if (!have_f) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const f32x4 la = *(const f32x4 *)(l2a + 32 * ks + 8 * G);
          const f32x4 lb = *(const f32x4 *)(l2a + 32 * ks + 8 * G + 4);
          const float l2e[8] = {la[0], la[1], la[2], la[3], lb[0], lb[1], lb[2], lb[3]};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            fi[ks][e] = fast_exp2((float)(row + 1) * l2e[e]);
            ft[ks][e] = fast_exp2((float)(row - CH_PIVOT) * l2e[e]);
          }
        }
        have_f = true;
      }
      bf16x8 qi[4], qt[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 qv = __builtin_bit_cast(bf16x8, qn[sl][ks]);
        float vi[8], vt[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          vi[e] = (float)qv[e] * fi[ks][e];
          vt[e] = (float)qv[e] * ft[ks][e];
        }
        qi[ks] = cvt8(vi);
        qt[ks] = cvt8(vt);
      }
      ch_issue_q(qn[sl], p, h, n2.valid ? n2 : c, w, i16, G);
      f32x4 acc[8];
      // inter term: O^T = S^T (Q (.) alpha^(row+1))^T
#pragma unroll
      for (int jt = 0; jt < 8; ++jt) {
        acc[jt] = (f32x4){};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc[jt] = mma16(lds_ld<bf16x8>((st ^ (ks << 6)) + 4096 * jt), qi[ks], acc[jt]);
      }
      // intra term over 32-key steps kp <= w / 2: P^T = K~ Q~^T for keys
      // 32 kp + (0..15) (p0) and 32 kp + 16 + (0..15) (p1), masked to
      // key <= row, then O^T += V^T P^T.
      for (int kp = 0; kp <= (w >> 1); ++kp) {
        const unsigned kb = kbase + 32 * kp * KV_ROW + kq;
        f32x4 p0 = {}, p1 = {};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          p0 = mma16(lds_ld<bf16x8>(kb ^ (ks << 6)), qt[ks], p0);
          p1 = mma16(lds_ld<bf16x8>((kb ^ (ks << 6)) + 16 * KV_ROW), qt[ks], p1);
        }
        const int n0 = row - (32 * kp + 4 * G), nn1 = n0 - 16;
        float pw[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pw[r] = (n0 >= r) ? p0[r] : 0.f;
          pw[4 + r] = (nn1 >= r) ? p1[r] : 0.f;
        }
        const bf16x8 pb = cvt8(pw);
        const unsigned vb = vbase + 32 * kp * KV_ROW + vq;
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
          const unsigned va = vb ^ (jt << 5);
          acc[jt] = mma16(tr_read8u(va, va + 16 * KV_ROW), pb, acc[jt]);
        }
      }
      __syncthreads();  // B: this chunk's K~, V and S^T reads are done
      {
        // acc[jt] register r: feature 16 jt + 4 G + r of chunk row `row`.
        // Staged in this wave's 16 rows of the output tile, then stored as
        // whole rows (16 lanes x 16 bytes per row; partial-line streaming
        // stores would cost HBM write efficiency) through a buffer whose
        // range ends with row L - 1.
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
          const bf16x4 o4 = {(bf16)acc[jt][0], (bf16)acc[jt][1], (bf16)acc[jt][2],
                             (bf16)acc[jt][3]};
          *(bf16x4 *)(Os + kv_off(row, (16 * jt + 4 * G) * 2)) = o4;
        }
        const int L = (int)(c.c1 - c.c0);
        const int rsb = (int)(m.rs * 2);
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (bf16 *)p.out + m.row_base<false>(h, c.j) + c.c0 * m.rs, 0, (L - 1) * rsb + D * 2,
            kRawBufferWord3);
        const int c16 = ln.lane & 15;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int r = 16 * w + 4 * it + (ln.lane >> 4);
          const u32x4 x = *(const u32x4 *)(Os + kv_off(r, 16 * c16));
          const int o = r < L ? r * rsb + 16 * c16 : (int)0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b128(x, rsrc, o, 0, kCpolNT);
        }
      }
      return n1.valid;
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    while (true) {
      if (!step(S0{}, cur, nxt)) break;
      cur = nxt;
      nxt = next_chunk<false>(m, cur, b, TC);
      if (!step(S1{}, cur, nxt)) break;
      cur = nxt;
      nxt = next_chunk<false>(m, cur, b, TC);
    }
  } else {
    const int u = ln.w, l32 = ln.l32, g = ln.g, lane = ln.lane, ts = ln.ts;
    float l2f[8], kf[4][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) l2f[e] = log2f(alpha[8 * (ts & 15) + e]);
    ch_tile_factors(kf, l2f, ts);
    const float l2ch = log2f(alpha[32 * u + l32]);  // this lane's A-operand channel
    float l2row[16];  // accumulator register r: state row 32u + 8(r/4) + 4g + r%4
#pragma unroll
    for (int r = 0; r < 16; ++r) l2row[r] = log2f(alpha[32 * u + 8 * (r >> 2) + 4 * g + (r & 3)]);
    float gam_full[16];  // alpha^TC of those rows (a whole chunk's state decay)
#pragma unroll
    for (int r = 0; r < 16; ++r) gam_full[r] = fast_exp2((float)TC * l2row[r]);
    f32x16 S[4];
    const float *s0 = p.ws ? p.ws + ((int64_t)s * p.r_split * H + h) * DD
                           : (p.init ? p.init + ((int64_t)cur.j * H + h) * DD : nullptr);
    load_state(S, s0, u, l32, g);
    // K/V two chunks ahead in two register sets (unconditional loads, as
    // on the output side).
    ChTiles t[2];
    Cursor nxt = next_chunk<false>(m, cur, b, TC);
    ch_load_tiles(t[0], p, h, cur, ts);
    ch_load_tiles(t[1], p, h, nxt.valid ? nxt : cur, ts);
    ch_store_tiles(Ks, Vs, t[0], (int)(cur.c1 - cur.c0), kf, ts);
    write_st(STs, S, u, l32, g);
    // One chunk: the tiles of c are in LDS and set sl^1 holds chunk n1;
    // set sl (already stored) is reloaded with chunk c + 2.
    auto step = [&](auto slot_c, const Cursor &c, const Cursor &n1) -> bool {
      constexpr int sl = decltype(slot_c)::value;
      const Cursor n2 = n1.valid ? next_chunk<false>(m, n1, b, TC) : n1;
      __syncthreads();  // A
      ch_load_tiles(t[sl], p, h, n2.valid ? n2 : c, ts);
      const int L = (int)(c.c1 - c.c0);
      const bool seq_done = (c.c1 == c.seq_end);
      const bool new_piece = n1.valid && (n1.c0 >= c.pend);
      if ((n1.valid && !new_piece) || (seq_done && p.fin)) {
        // alpha^L per state row: a whole chunk's factors are taken once
        if (L == TC) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) S[nt][r] *= gam_full[r];
        } else {
          float gam[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) gam[r] = fast_exp2((float)L * l2row[r]);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) S[nt][r] *= gam[r];
        }
        ch_state_update(S, Ks, Vs, fast_exp2((float)(L - 1 - CH_PIVOT) * l2ch), u, lane);
        if (seq_done && p.fin) store_state(p.fin + ((int64_t)c.j * H + h) * DD, S, u, l32, g);
      }
      __syncthreads();  // B
      if (!n1.valid) return false;
      if (new_piece) {
        load_state(S, p.init ? p.init + ((int64_t)n1.j * H + h) * DD : nullptr, u, l32, g);
        // Waited for here, on this rare path: left to the compiler, the wait
        // for these loads would land after the join, on every chunk, and
        // take the prefetched tiles with it.
        vm_wait<0>();
      }
      ch_store_tiles(Ks, Vs, t[sl ^ 1], (int)(n1.c1 - n1.c0), kf, ts);
      write_st(STs, S, u, l32, g);
      return true;
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    while (true) {
      if (!step(S0{}, cur, nxt)) break;
      cur = nxt;
      nxt = next_chunk<false>(m, cur, b, TC);
      if (!step(S1{}, cur, nxt)) break;
      cur = nxt;
      nxt = next_chunk<false>(m, cur, b, TC);
    }
  }
}

}  // namespace mfma
}  // namespace la
