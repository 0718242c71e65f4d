// Small kernels around the backward pass.  The gradients themselves come
// from three passes of the prefill kernels (see lightning_attn_bwd in
// lightning_attn.hip): with G_t = dL/dS_t, the gradient of the state,
//   dq_t = do_t S_t^T                      causal pass  (q, k, v) <- (do, v, k)
//   dv_t = k_t G_t,  dk_t = v_t G_t^T      time-reversed passes
//                                          (q, k, v) <- (k, q, do) and (v, do, q)
// G_t = q_t^T do_t + lambda G_{t+1} runs backwards from dS_fin, so a reversed
// pass starts from dS_fin / lambda (its kernels decay an initial state once
// more than G needs), and dS_init = lambda G_0 = lambda x (the dv pass's final
// state).  These kernels form those states, and (for the vector-ALU path,
// which runs the dk pass on its own) transpose the dv pass's segment entering
// states into the dk pass's (G and G^T share segments); on MFMA the dv and dk
// passes run as one (prefill_dkdv_kernel), the dk side reading G transposed.
#pragma once

#include "la_common.h"

namespace la {

// g = dfin / lambda, per (sequence, head) u and element e of the states.
__global__ __launch_bounds__(256) void bwd_scale_kernel(const float *dfin, const float *decay,
                                                        int H, int d, float *g) {
  const int u = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  const int dd = d * d;
  if (e >= dd) return;
  const int64_t o = (int64_t)u * dd + e;
  g[o] = dfin[o] / decay[u % H];
}

// dst[u] = f_u src[u']^T for the n = grid.x states u, with u' = (u / H) R H
// + u % H (state u' of a [.][R][H] array: R = 1 for a plain [.][H] array)
// and f_u = 1 / lambda_{u % H} when inv_decay, else 1.  32 x 32 tiles through
// LDS, so that both the reads and the writes are whole rows.
__global__ __launch_bounds__(256) void transpose_states_kernel(const float *src, int R, int H,
                                                               int d, const float *decay,
                                                               bool inv_decay, float *dst) {
  __shared__ float tile[32][33];
  const int u = blockIdx.x;
  const int bi = blockIdx.y * 32, bj = blockIdx.z * 32;  // source rows, source columns
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const int64_t dd = (int64_t)d * d;
  const float *S = src + ((int64_t)(u / H) * R * H + u % H) * dd;
  float *T = dst + (int64_t)u * dd;
  const float f = inv_decay ? 1.f / decay[u % H] : 1.f;
  for (int k = ty; k < 32; k += 8) tile[k][tx] = S[(int64_t)(bi + k) * d + bj + tx];
  __syncthreads();
  for (int k = ty; k < 32; k += 8) T[(int64_t)(bj + k) * d + bi + tx] = f * tile[tx][k];
}

// dinit = scale_h * src (src NULL: zero); scale_h = lambda_h, or 1 when
// use_decay is false (an empty sequence passes dS_fin through unchanged).
__global__ __launch_bounds__(256) void bwd_dinit_kernel(const float *src, const float *decay,
                                                        int H, int d, bool use_decay,
                                                        float *dinit) {
  const int u = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  const int dd = d * d;
  if (e >= dd) return;
  const int64_t o = (int64_t)u * dd + e;
  const float s = use_decay ? decay[u % H] : 1.f;
  dinit[o] = src ? s * src[o] : 0.f;
}

}  // namespace la
