/* A plain C99 program that drives the library on the GPU through its C ABI
 * alone (HIP runtime calls for memory, no Python): a bf16 prefill of
 * B=2, H=3, N=700, d=128 with an initial state and the library's own
 * workspace query, then one decode step from the final states.  Inputs come
 * from a seeded xorshift generator; the reference is the double-precision
 * oracle (liboracle.so, oracle_fwd_f64 and oracle_decode_f64) on the same
 * bf16-rounded values.  Built by the package build; run by
 * tests/test_c_caller_gpu.py.  Prints the relative errors and exits 0 when
 * they are within the bf16 tolerance (2e-2). */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lightning_attn.h"

/* The oracle's entry points (oracle/oracle.c). */
int oracle_fwd_f64(const float *q, const float *k, const float *v, const float *decay, int B,
                   int H, int64_t N, int d, const double *init, double *out, double *fin,
                   int nthreads);
int oracle_decode_f64(const float *q, const float *k, const float *v, const float *decay, int B,
                      int H, int d, double *state, double *out, int nthreads);

#define CHECK_HIP(x)                                                  \
  do {                                                                \
    hipError_t e_ = (x);                                              \
    if (e_ != hipSuccess) {                                           \
      printf("HIP error %s at %s\n", hipGetErrorString(e_), #x);      \
      exit(2);                                                        \
    }                                                                 \
  } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;

static double uniform01(void) {
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return ((rng * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0) + 1e-300;
}

static double normal(void) {
  return sqrt(-2.0 * log(uniform01())) * cos(6.283185307179586 * uniform01());
}

/* float -> bf16 bits, round to nearest even (finite inputs). */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* n values N(0, 1) / sqrt(d), as bf16 bits and as the floats they hold. */
static void fill(uint16_t *b, float *f, size_t n, int d) {
  for (size_t i = 0; i < n; ++i) {
    b[i] = to_bf16((float)(normal() / sqrt((double)d)));
    f[i] = from_bf16(b[i]);
  }
}

static double rel_err_bf16(const uint16_t *x, const double *ref, size_t n) {
  double num = 0.0, den = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double a = from_bf16(x[i]);
    if (!isfinite(a)) return INFINITY;
    num = fmax(num, fabs(a - ref[i]));
    den = fmax(den, fabs(ref[i]));
  }
  return den > 0 ? num / den : num;
}

static double rel_err_f32(const float *x, const double *ref, size_t n) {
  double num = 0.0, den = 0.0;
  for (size_t i = 0; i < n; ++i) {
    if (!isfinite(x[i])) return INFINITY;
    num = fmax(num, fabs(x[i] - ref[i]));
    den = fmax(den, fabs(ref[i]));
  }
  return den > 0 ? num / den : num;
}

int main(void) {
  const int B = 2, H = 3, d = 128, block = 128;
  const int64_t N = 700;
  const size_t nt = (size_t)B * H * N * d, ns = (size_t)B * H * d * d, nd = (size_t)B * H * d;
  uint16_t *hq = malloc(nt * 2), *hk = malloc(nt * 2), *hv = malloc(nt * 2), *ho = malloc(nt * 2);
  float *fq = malloc(nt * 4), *fk = malloc(nt * 4), *fv = malloc(nt * 4);
  float *init = malloc(ns * 4), *fin = malloc(ns * 4);
  double *init_d = malloc(ns * 8), *out_ref = malloc(nt * 8), *fin_ref = malloc(ns * 8);
  float decay[3];
  if (!hq || !hk || !hv || !ho || !fq || !fk || !fv || !init || !fin || !init_d || !out_ref ||
      !fin_ref) {
    printf("host allocation failed\n");
    return 2;
  }
  fill(hq, fq, nt, d);
  fill(hk, fk, nt, d);
  fill(hv, fv, nt, d);
  for (size_t i = 0; i < ns; ++i) {
    init[i] = (float)(0.1 * normal());
    init_d[i] = init[i];
  }
  for (int h = 0; h < H; ++h) decay[h] = (float)exp(-pow(2.0, -8.0 * (h + 1) / H));

  void *dq, *dk, *dv, *dout, *dws = NULL;
  float *ddecay, *dinit, *dfin;
  CHECK_HIP(hipMalloc(&dq, nt * 2));
  CHECK_HIP(hipMalloc(&dk, nt * 2));
  CHECK_HIP(hipMalloc(&dv, nt * 2));
  CHECK_HIP(hipMalloc(&dout, nt * 2));
  CHECK_HIP(hipMalloc((void **)&ddecay, sizeof(decay)));
  CHECK_HIP(hipMalloc((void **)&dinit, ns * 4));
  CHECK_HIP(hipMalloc((void **)&dfin, ns * 4));
  CHECK_HIP(hipMemcpy(dq, hq, nt * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dk, hk, nt * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, hv, nt * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(ddecay, decay, sizeof(decay), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dinit, init, ns * 4, hipMemcpyHostToDevice));
  /* a segment length that cuts the sequences (the scan runs) */
  const int64_t seg = 256;
  const size_t ws = lightning_attn_fwd_workspace_size(B, H, N, d, block, LA_BF16, seg);
  if (ws) CHECK_HIP(hipMalloc(&dws, ws));

  la_status st = lightning_attn_fwd(dq, dk, dv, ddecay, B, H, N, d, block, LA_BF16, dinit, dout,
                                    dfin, seg, dws, ws, NULL);
  if (st != LA_OK) {
    printf("lightning_attn_fwd: %s\n", lightning_attn_status_string(st));
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(ho, dout, nt * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(fin, dfin, ns * 4, hipMemcpyDeviceToHost));
  oracle_fwd_f64(fq, fk, fv, decay, B, H, N, d, init_d, out_ref, fin_ref, 0);
  const double eo = rel_err_bf16(ho, out_ref, nt), ef = rel_err_f32(fin, fin_ref, ns);
  printf("prefill B=%d H=%d N=%lld d=%d workspace %zu B: out %.3e final state %.3e\n", B, H,
         (long long)N, d, ws, eo, ef);

  /* One decode step from the final states (state updated in place). */
  uint16_t *hdq = malloc(nd * 2), *hdk = malloc(nd * 2), *hdv = malloc(nd * 2),
           *hdo = malloc(nd * 2);
  float *fdq = malloc(nd * 4), *fdk = malloc(nd * 4), *fdv = malloc(nd * 4);
  double *dout_ref = malloc(nd * 8);
  fill(hdq, fdq, nd, d);
  fill(hdk, fdk, nd, d);
  fill(hdv, fdv, nd, d);
  void *ddq, *ddk, *ddv, *ddo;
  CHECK_HIP(hipMalloc(&ddq, nd * 2));
  CHECK_HIP(hipMalloc(&ddk, nd * 2));
  CHECK_HIP(hipMalloc(&ddv, nd * 2));
  CHECK_HIP(hipMalloc(&ddo, nd * 2));
  CHECK_HIP(hipMemcpy(ddq, hdq, nd * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(ddk, hdk, nd * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(ddv, hdv, nd * 2, hipMemcpyHostToDevice));
  st = lightning_attn_decode(ddq, ddk, ddv, ddecay, dfin, ddo, B, H, d, LA_BF16, NULL);
  if (st != LA_OK) {
    printf("lightning_attn_decode: %s\n", lightning_attn_status_string(st));
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(hdo, ddo, nd * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(fin, dfin, ns * 4, hipMemcpyDeviceToHost));
  oracle_decode_f64(fdq, fdk, fdv, decay, B, H, d, fin_ref, dout_ref, 0);
  const double edo = rel_err_bf16(hdo, dout_ref, nd), eds = rel_err_f32(fin, fin_ref, ns);
  printf("decode: out %.3e state %.3e\n", edo, eds);

  const int ok = eo <= 2e-2 && ef <= 2e-2 && edo <= 2e-2 && eds <= 2e-2;
  printf("%s\n", ok ? "PASS" : "FAIL");
  return ok ? 0 : 1;
}
