// Small kernels around the backward pass.  The gradients themselves come
// from three passes of the prefill kernels (see lightning_attn_bwd in
// lightning_attn.hip): with G_t = dL/dS_t, the gradient of the state,
//   dq_t = do_t S_t^T                      causal pass  (q, k, v) <- (do, v, k)
//   dv_t = k_t G_t,  dk_t = v_t G_t^T      time-reversed passes
//                                          (q, k, v) <- (k, q, do) and (v, do, q)
// G_t = q_t^T do_t + lambda G_{t+1} runs backwards from dS_fin, so a reversed
// pass starts from dS_fin / lambda (its kernels decay an initial state once
// more than G needs), and dS_init = lambda G_0 = lambda x (the dv pass's final
// state).  These kernels form those states.
#pragma once

#include "la_common.h"

namespace la {

// Per (sequence, head) u and element e = (i, j) of the d x d states:
//   initT = init^T;  g = dfin / lambda;  gT = g^T   (each when its source is given).
__global__ __launch_bounds__(256) void bwd_prep_kernel(const float *init, const float *dfin,
                                                       const float *decay, int H, int d,
                                                       float *initT, float *g, float *gT) {
  const int u = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  const int dd = d * d;
  if (e >= dd) return;
  const int i = e / d, j = e - (e / d) * d;
  const int64_t o = (int64_t)u * dd;
  if (init) initT[o + (int64_t)j * d + i] = init[o + e];
  if (dfin) {
    const float x = dfin[o + e] / decay[u % H];
    g[o + e] = x;
    gT[o + (int64_t)j * d + i] = x;
  }
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
