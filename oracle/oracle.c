/*
 * Lightning attention CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py
 * may load this library.  The product path (the HIP library and its Python
 * binding) never calls it and shares no code with it.
 *
 * What it computes (causal linear attention with a per-head scalar decay,
 * no normalisation, no activation, no gate):
 *
 *   MiniMax-01 technical report (full Chinese translation, blog.csdn.net),
 *   section 2.2.1 "Lightning Attention":
 *     - the causal left product (eq. 4): O = [(Q K^T) (.) M] V with
 *       M[t][s] = 1 when t >= s, else 0 (the diagonal is included);
 *     - the right-product recurrence (eq. 5): kv_t = kv_{t-1} + k_t^T v_t,
 *       o_t = q_t kv_t, with kv_0 = 0;
 *     - normalisation, SiLU and the gate are deliberately left out of the
 *       derivation there, so they are left out here too.
 *   Section 2.2.4 (eq. 12) gives lightning attention's recurrent (RNN)
 *   form; section 3.2.2 (Fig. 12) initialises a diagonal decay matrix; the
 *   K3 reading notes (cutenote.app, "solution 1: add a position decay term")
 *   name the RetNet-style decay.  With a per-head decay lambda these read
 *
 *     S_t = lambda * S_{t-1} + k_t^T v_t          (S_t is d x d, S_{-1} = S_init)
 *     o_t = q_t S_t                               (o_t[j] = sum_i q_t[i] S_t[i][j])
 *
 *   and, unrolled (the decayed left product),
 *
 *     o_t = sum_{s<=t} lambda^(t-s) (q_t . k_s) v_s + lambda^(t+1) q_t S_init.
 *
 * Arithmetic is IEEE double throughout.  Inputs arrive as float32 arrays: the
 * exact values handed to the GPU (bf16 values widen to float32 exactly); the
 * decay arrives as the float32 lambda the GPU gets, widened to double.
 *
 * Layouts (row-major, d fastest):
 *   fixed length : q, k, v, out  [B][H][N][d];  states [B][H][d][d]
 *   packed varlen: q, k, v, out  [H][total][d]; sequence j occupies tokens
 *                  cu[j] .. cu[j+1]-1 of every head; states [S][H][d][d]
 *   states are S[i][j] with i the key feature and j the value feature.
 *
 * Every function is threaded over independent (sequence, head) units with
 * pthreads; nthreads <= 0 means "all CPUs this process may run on".
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ---------------------------------------------------------------- threads */

typedef void (*unit_fn)(void *ctx, int64_t unit);

typedef struct {
  unit_fn fn;
  void *ctx;
  int64_t n_units;
  int64_t next;
  pthread_mutex_t lock;
} pool_t;

static void *pool_worker(void *arg) {
  pool_t *p = (pool_t *)arg;
  for (;;) {
    pthread_mutex_lock(&p->lock);
    int64_t u = p->next++;
    pthread_mutex_unlock(&p->lock);
    if (u >= p->n_units) break;
    p->fn(p->ctx, u);
  }
  return NULL;
}

int oracle_default_threads(void) {
  cpu_set_t set;
  CPU_ZERO(&set);
  if (sched_getaffinity(0, sizeof(set), &set) == 0) {
    int c = CPU_COUNT(&set);
    if (c > 0) return c;
  }
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

/* Runs fn(ctx, u) for u in [0, n_units); returns the thread count used. */
static int run_units(unit_fn fn, void *ctx, int64_t n_units, int nthreads) {
  if (nthreads <= 0) nthreads = oracle_default_threads();
  if ((int64_t)nthreads > n_units) nthreads = (int)(n_units > 0 ? n_units : 1);
  pool_t p;
  p.fn = fn;
  p.ctx = ctx;
  p.n_units = n_units;
  p.next = 0;
  pthread_mutex_init(&p.lock, NULL);
  if (nthreads <= 1) {
    pool_worker(&p);
  } else {
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int i = 0; i < nthreads; ++i)
      if (pthread_create(&tid[i], NULL, pool_worker, &p) == 0) ++started;
    if (started == 0) pool_worker(&p);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    free(tid);
    if (started > 0) nthreads = started; else nthreads = 1;
  }
  pthread_mutex_destroy(&p.lock);
  return nthreads;
}

/* ------------------------------------------------- one sequence, one head */

/* ORACLE_PLANT selects a deliberately wrong recurrence; it is only ever set
 * by the CPU test that checks the oracle's pins catch such mistakes.
 * 0 = correct; 1 = decay applied after the add; 2 = transposed outer product;
 * 3 = output read before the update; 4 = decay dropped; 5 = output contracts
 * the state's other index; 6 = prefix-state snapshots taken one token early. */
#ifndef ORACLE_PLANT
#define ORACLE_PLANT 0
#endif

/*
 * The recurrence (eq. 5 with the per-head decay) over n tokens of one head.
 * q, k, v point at row 0 of the sequence ([n][d], d fastest).  S (d*d) holds
 * the state entering the sequence and is left holding the state after its
 * last token.  out ([n][d]) may be NULL when only the state is wanted.
 */
static void recur_one(const float *q, const float *k, const float *v, double lam, int64_t n,
                      int d, double *S, double *out, double *orow) {
  for (int64_t t = 0; t < n; ++t) {
    const float *kt = k + t * d, *vt = v + t * d, *qt = q + t * d;
    /* S_t = lambda S_{t-1} + k_t^T v_t */
    if (ORACLE_PLANT == 3 && out) {
      for (int j = 0; j < d; ++j) orow[j] = 0.0;
      for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) orow[j] += (double)qt[i] * S[(int64_t)i * d + j];
    }
    for (int i = 0; i < d; ++i) {
      double ki = (double)kt[i];
      double *Si = S + (int64_t)i * d;
      for (int j = 0; j < d; ++j) {
        if (ORACLE_PLANT == 1) Si[j] = lam * (Si[j] + ki * (double)vt[j]);
        else if (ORACLE_PLANT == 2) Si[j] = lam * Si[j] + (double)kt[j] * (double)vt[i];
        else if (ORACLE_PLANT == 4) Si[j] = Si[j] + ki * (double)vt[j];
        else Si[j] = lam * Si[j] + ki * (double)vt[j];
      }
    }
    if (!out) continue;
    /* o_t = q_t S_t */
    if (ORACLE_PLANT != 3) {
      for (int j = 0; j < d; ++j) orow[j] = 0.0;
      for (int i = 0; i < d; ++i) {
        double qi = (double)qt[i];
        const double *Si = S + (int64_t)i * d;
        for (int j = 0; j < d; ++j) {
          if (ORACLE_PLANT == 5) orow[j] += qi * S[(int64_t)j * d + i];
          else orow[j] += qi * Si[j];
        }
      }
    }
    memcpy(out + t * d, orow, sizeof(double) * (size_t)d);
  }
}

/* ------------------------------------------------------ fixed-length fwd */

typedef struct {
  const float *q, *k, *v, *decay;
  int B, H, d;
  int64_t N;
  const double *init;
  double *out, *fin;
} fwd_ctx;

static void fwd_unit(void *vctx, int64_t u) {
  fwd_ctx *c = (fwd_ctx *)vctx;
  int d = c->d;
  int h = (int)(u % c->H);
  int64_t base = u * c->N * d;
  int64_t dd = (int64_t)d * d;
  double *S = (double *)malloc(sizeof(double) * (size_t)dd);
  double *orow = (double *)malloc(sizeof(double) * (size_t)d);
  if (c->init) memcpy(S, c->init + u * dd, sizeof(double) * (size_t)dd);
  else memset(S, 0, sizeof(double) * (size_t)dd);
  recur_one(c->q + base, c->k + base, c->v + base, (double)c->decay[h], c->N, d, S,
            c->out ? c->out + base : NULL, orow);
  if (c->fin) memcpy(c->fin + u * dd, S, sizeof(double) * (size_t)dd);
  free(orow);
  free(S);
}

/* Prefill over [B][H][N][d]; init may be NULL (zero state); out or fin may
 * be NULL.  Returns the number of threads used. */
int oracle_fwd_f64(const float *q, const float *k, const float *v, const float *decay, int B,
                   int H, int64_t N, int d, const double *init, double *out, double *fin,
                   int nthreads) {
  fwd_ctx c = {q, k, v, decay, B, H, d, N, init, out, fin};
  return run_units(fwd_unit, &c, (int64_t)B * H, nthreads);
}

/* ------------------------------------------------------------ varlen fwd */

typedef struct {
  const float *q, *k, *v, *decay;
  const int32_t *cu;
  int S, H, d;
  int64_t total;
  const double *init;
  double *out, *fin;
  int64_t snap_iv;         /* 0: no snapshots */
  const int32_t *snap_off; /* [S + 1] first snapshot row of each sequence */
  double *snaps;           /* [rows][H][d][d] */
} var_ctx;

static void var_unit(void *vctx, int64_t u) {
  var_ctx *c = (var_ctx *)vctx;
  int d = c->d;
  int64_t j = u / c->H;
  int h = (int)(u % c->H);
  int64_t t0 = c->cu[j], n = (int64_t)c->cu[j + 1] - c->cu[j];
  int64_t base = ((int64_t)h * c->total + t0) * d;
  int64_t dd = (int64_t)d * d;
  int64_t sidx = (j * c->H + h) * dd;
  double *S = (double *)malloc(sizeof(double) * (size_t)dd);
  double *orow = (double *)malloc(sizeof(double) * (size_t)d);
  if (c->init) memcpy(S, c->init + sidx, sizeof(double) * (size_t)dd);
  else memset(S, 0, sizeof(double) * (size_t)dd);
  /* The recurrence runs in steps of snap_iv tokens (one step without
   * snapshots); after each full step the state is the prefix state after
   * that many tokens of the sequence, and is copied out. */
  int64_t step = c->snap_iv > 0 ? c->snap_iv : (n > 0 ? n : 1);
  for (int64_t t = 0, m = 0; t < n; t += step) {
    int64_t len = n - t < step ? n - t : step;
    int snap = c->snap_iv > 0 && len == step;
    /* (plant 6 takes the snapshot one token short of its point) */
    int64_t first = (ORACLE_PLANT == 6 && snap) ? len - 1 : len;
    recur_one(c->q + base + t * d, c->k + base + t * d, c->v + base + t * d,
              (double)c->decay[h], first, d, S, c->out ? c->out + base + t * d : NULL, orow);
    if (snap) {
      int64_t row = (int64_t)c->snap_off[j] + m++;
      memcpy(c->snaps + (row * c->H + h) * dd, S, sizeof(double) * (size_t)dd);
    }
    if (first < len)
      recur_one(c->q + base + (t + first) * d, c->k + base + (t + first) * d,
                c->v + base + (t + first) * d, (double)c->decay[h], len - first, d, S,
                c->out ? c->out + base + (t + first) * d : NULL, orow);
  }
  if (c->fin) memcpy(c->fin + sidx, S, sizeof(double) * (size_t)dd);
  free(orow);
  free(S);
}

/* Packed variable-length prefill: the state starts afresh (from init[j] or
 * zero) at every sequence start, as data packing requires (MiniMax-01 report,
 * section 3.2 "data packing"; section 3.2.2 varlen for LASP+). */
int oracle_fwd_varlen_f64(const float *q, const float *k, const float *v, const float *decay,
                          const int32_t *cu_seqlens, int num_seqs, int H, int64_t total, int d,
                          const double *init, double *out, double *fin, int nthreads) {
  var_ctx c = {q, k, v, decay, cu_seqlens, num_seqs, H, d, total, init, out, fin, 0, NULL, NULL};
  return run_units(var_unit, &c, (int64_t)num_seqs * H, nthreads);
}

/* Packed prefill that also keeps prefix states (the K3 reading notes'
 * inference-engine part: one prefix state per block, since a linear-attention
 * state is rewritten at every token): snapshot m = 1, 2, ... of sequence j
 * is the state after its first m * snap_iv tokens, S_{m snap_iv - 1} of the
 * recurrence above (so it includes the sequence's initial state), stored at
 * row snap_off[j] + m - 1 of snaps ([rows][H][d][d]).  snap_iv >= 1. */
int oracle_fwd_varlen_snap_f64(const float *q, const float *k, const float *v, const float *decay,
                               const int32_t *cu_seqlens, int num_seqs, int H, int64_t total,
                               int d, const double *init, double *out, double *fin,
                               int64_t snap_iv, const int32_t *snap_off, double *snaps,
                               int nthreads) {
  var_ctx c = {q, k, v, decay, cu_seqlens, num_seqs, H, d, total, init, out, fin,
               snap_iv, snap_off, snaps};
  return run_units(var_unit, &c, (int64_t)num_seqs * H, nthreads);
}

/* ------------------------------------------------- channel-wise decay */

/*
 * The channel-wise variant (K3 reading notes, "gated DeltaNet": the scalar
 * decay replaced by one decay per channel, strictly more general since equal
 * channels give back the scalar form; here without the delta rule): head h
 * has a decay alpha[h][i] for every key channel i, and
 *
 *   S_t[i][j] = alpha_i S_{t-1}[i][j] + k_t[i] v_t[j],     o_t = q_t S_t,
 *
 * i.e. o_t[j] = sum_{s<=t} sum_i q_t[i] alpha_i^(t-s) k_s[i] v_s[j]
 *             + sum_i q_t[i] alpha_i^(t+1) S_init[i][j].
 * alpha is [H][d] float32 (widened to double); layout as oracle_fwd_f64.
 */
#ifndef ORACLE_PLANT_CH
#define ORACLE_PLANT_CH 0 /* 1 = decay indexed by the value channel (a planted mistake) */
#endif

typedef struct {
  const float *q, *k, *v, *alpha;
  int H, d;
  int64_t N;
  const double *init;
  double *out, *fin;
} ch_ctx;

static void ch_unit(void *vctx, int64_t u) {
  ch_ctx *c = (ch_ctx *)vctx;
  int d = c->d, h = (int)(u % c->H);
  int64_t N = c->N, dd = (int64_t)d * d, base = u * N * d;
  const float *al = c->alpha + (int64_t)h * d;
  double *S = (double *)malloc(sizeof(double) * (size_t)dd);
  if (c->init) memcpy(S, c->init + u * dd, sizeof(double) * (size_t)dd);
  else memset(S, 0, sizeof(double) * (size_t)dd);
  for (int64_t t = 0; t < N; ++t) {
    const float *qt = c->q + base + t * d, *kt = c->k + base + t * d, *vt = c->v + base + t * d;
    for (int i = 0; i < d; ++i) {
      double a = (double)al[i], ki = (double)kt[i];
      for (int j = 0; j < d; ++j) {
        if (ORACLE_PLANT_CH == 1) a = (double)al[j];
        S[(int64_t)i * d + j] = a * S[(int64_t)i * d + j] + ki * (double)vt[j];
      }
    }
    if (c->out) {
      double *o = c->out + base + t * d;
      for (int j = 0; j < d; ++j) o[j] = 0.0;
      for (int i = 0; i < d; ++i) {
        double qi = (double)qt[i];
        for (int j = 0; j < d; ++j) o[j] += qi * S[(int64_t)i * d + j];
      }
    }
  }
  if (c->fin) memcpy(c->fin + u * dd, S, sizeof(double) * (size_t)dd);
  free(S);
}

int oracle_fwd_chdecay_f64(const float *q, const float *k, const float *v, const float *alpha,
                           int B, int H, int64_t N, int d, const double *init, double *out,
                           double *fin, int nthreads) {
  ch_ctx c = {q, k, v, alpha, H, d, N, init, out, fin};
  return run_units(ch_unit, &c, (int64_t)B * H, nthreads);
}

/* -------------------------------------------------------------- backward */

/*
 * Gradients of the prefill (training).  The pages give no backward
 * derivation, so it is the derivative of the recurrence above, taken by
 * hand: with do_t = dL/do_t and dS_fin = dL/dS_{N-1},
 *
 *   G_t  = dL/dS_t (through o_t and every later state)
 *        = q_t^T do_t + lambda G_{t+1},    G_{N-1} = q_{N-1}^T do_{N-1} + dS_fin
 *   dq_t = do_t S_t^T            (dq_t[i] = sum_j do_t[j] S_t[i][j], S_t from the recurrence)
 *   dk_t = v_t G_t^T             (dk_t[i] = sum_j G_t[i][j] v_t[j])
 *   dv_t = k_t G_t               (dv_t[j] = sum_i k_t[i] G_t[i][j])
 *   dS_init = lambda G_0         (dS_fin itself when N == 0)
 *
 * Layout as oracle_fwd_f64; dfin, init and dinit may be NULL (zero / not
 * wanted).
 */
#ifndef ORACLE_PLANT_BWD
#define ORACLE_PLANT_BWD 0
#endif

typedef struct {
  const float *q, *k, *v, *decay, *dout;
  int H, d;
  int64_t N;
  const double *dfin, *init;
  double *dq, *dk, *dv, *dinit;
} bwd_ctx;

static void bwd_unit(void *vctx, int64_t u) {
  bwd_ctx *c = (bwd_ctx *)vctx;
  int d = c->d;
  int64_t N = c->N, dd = (int64_t)d * d, base = u * N * d;
  double lam = (double)c->decay[u % c->H];
  const float *q = c->q + base, *k = c->k + base, *v = c->v + base, *g = c->dout + base;
  double *S = (double *)malloc(sizeof(double) * (size_t)dd);
  /* dq: the forward recurrence, contracting each state with do_t */
  if (c->init) memcpy(S, c->init + u * dd, sizeof(double) * (size_t)dd);
  else memset(S, 0, sizeof(double) * (size_t)dd);
  for (int64_t t = 0; t < N; ++t) {
    const float *kt = k + t * d, *vt = v + t * d, *gt = g + t * d;
    if (ORACLE_PLANT_BWD == 3) { /* reads the state before token t's update */
      for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int j = 0; j < d; ++j) acc += (double)gt[j] * S[(int64_t)i * d + j];
        c->dq[base + t * d + i] = acc;
      }
    }
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j)
        S[(int64_t)i * d + j] = lam * S[(int64_t)i * d + j] + (double)kt[i] * (double)vt[j];
    if (ORACLE_PLANT_BWD != 3) {
      for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int j = 0; j < d; ++j) acc += (double)gt[j] * S[(int64_t)i * d + j];
        c->dq[base + t * d + i] = acc;
      }
    }
  }
  /* dk, dv: G backwards from the last token */
  double *G = S;
  if (c->dfin) memcpy(G, c->dfin + u * dd, sizeof(double) * (size_t)dd);
  else memset(G, 0, sizeof(double) * (size_t)dd);
  for (int64_t t = N - 1; t >= 0; --t) {
    const float *qt = q + t * d, *kt = k + t * d, *vt = v + t * d, *gt = g + t * d;
    double f = (t == N - 1) ? 1.0 : lam;
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j)
        G[(int64_t)i * d + j] = f * G[(int64_t)i * d + j] + (double)qt[i] * (double)gt[j];
    for (int i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int j = 0; j < d; ++j)
        acc += (ORACLE_PLANT_BWD == 1 ? G[(int64_t)j * d + i] : G[(int64_t)i * d + j]) *
               (double)vt[j];
      c->dk[base + t * d + i] = acc;
    }
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += (double)kt[i] * G[(int64_t)i * d + j];
      c->dv[base + t * d + j] = acc;
    }
  }
  if (c->dinit) {
    double f = (N > 0 && ORACLE_PLANT_BWD != 2) ? lam : 1.0;
    for (int64_t e = 0; e < dd; ++e) c->dinit[u * dd + e] = f * G[e];
  }
  free(S);
}

int oracle_bwd_f64(const float *q, const float *k, const float *v, const float *decay,
                   const float *dout, const double *dfin, const double *init, int B, int H,
                   int64_t N, int d, double *dq, double *dk, double *dv, double *dinit,
                   int nthreads) {
  bwd_ctx c = {q, k, v, decay, dout, H, d, N, dfin, init, dq, dk, dv, dinit};
  return run_units(bwd_unit, &c, (int64_t)B * H, nthreads);
}

/* ---------------------------------------------------------------- decode */

typedef struct {
  const float *q, *k, *v, *decay;
  int H, d;
  double *state, *out;
} dec_ctx;

static void dec_unit(void *vctx, int64_t u) {
  dec_ctx *c = (dec_ctx *)vctx;
  int d = c->d;
  int h = (int)(u % c->H);
  double *orow = (double *)malloc(sizeof(double) * (size_t)d);
  recur_one(c->q + u * d, c->k + u * d, c->v + u * d, (double)c->decay[h], 1, d,
            c->state + u * (int64_t)d * d, c->out + u * d, orow);
  free(orow);
}

/* One recurrent (RNN-form) step for [B][H] heads: state <- lambda state +
 * k^T v, then out = q state (the output reads the updated state, so decoding
 * token t from the state after t-1 tokens reproduces prefill row t).
 * state is [B][H][d][d] double, updated in place; q, k, v, out are [B][H][d]. */
int oracle_decode_f64(const float *q, const float *k, const float *v, const float *decay, int B,
                      int H, int d, double *state, double *out, int nthreads) {
  dec_ctx c = {q, k, v, decay, H, d, state, out};
  return run_units(dec_unit, &c, (int64_t)B * H, nthreads);
}

/* ------------------------------------------------ decayed left product */

typedef struct {
  const float *q, *k, *v, *decay;
  int H, d;
  int64_t N;
  const double *init;
  double *out, *fin;
} bf_ctx;

static void bf_unit(void *vctx, int64_t u) {
  bf_ctx *c = (bf_ctx *)vctx;
  int d = c->d;
  int64_t N = c->N;
  double lam = (double)c->decay[u % c->H];
  int64_t base = u * N * d, dd = (int64_t)d * d;
  const float *q = c->q + base, *k = c->k + base, *v = c->v + base;
  const double *S0 = c->init ? c->init + u * dd : NULL;
  for (int64_t t = 0; t < N; ++t) {
    double *o = c->out + base + t * d;
    for (int j = 0; j < d; ++j) o[j] = 0.0;
    /* masked, decayed scores: [(Q K^T) (.) M_lambda]_{t,s} for s <= t */
    for (int64_t s = 0; s <= t; ++s) {
      double score = 0.0;
      for (int i = 0; i < d; ++i) score += (double)q[t * d + i] * (double)k[s * d + i];
      score *= pow(lam, (double)(t - s));
      for (int j = 0; j < d; ++j) o[j] += score * (double)v[s * d + j];
    }
    if (S0) {
      double a = pow(lam, (double)(t + 1));
      for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) o[j] += a * (double)q[t * d + i] * S0[i * d + j];
    }
  }
  if (c->fin) {
    double *S = c->fin + u * dd;
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        double acc = S0 ? pow(lam, (double)N) * S0[i * d + j] : 0.0;
        for (int64_t s = 0; s < N; ++s)
          acc += pow(lam, (double)(N - 1 - s)) * (double)k[s * d + i] * (double)v[s * d + j];
        S[i * d + j] = acc;
      }
  }
}

/* The left-product form (eq. 4 with the decay folded into the mask):
 * O(N^2 d) per head, for small inputs only.  Same layout as oracle_fwd_f64;
 * out must not be NULL. */
int oracle_bruteforce_f64(const float *q, const float *k, const float *v, const float *decay,
                          int B, int H, int64_t N, int d, const double *init, double *out,
                          double *fin, int nthreads) {
  bf_ctx c = {q, k, v, decay, H, d, N, init, out, fin};
  return run_units(bf_unit, &c, (int64_t)B * H, nthreads);
}

/* --------------------------------------------- sampled outputs, large N */

typedef struct {
  const float *q, *k, *v;
  double lam;
  int d;
  const int64_t *rows;
  const double *init;
  double *out;
} row_ctx;

static void row_unit(void *vctx, int64_t u) {
  row_ctx *c = (row_ctx *)vctx;
  int d = c->d;
  int64_t t = c->rows[u];
  const float *qt = c->q + t * d;
  double *o = c->out + u * d;
  for (int j = 0; j < d; ++j) o[j] = 0.0;
  for (int64_t s = 0; s <= t; ++s) {
    double score = 0.0;
    for (int i = 0; i < d; ++i) score += (double)qt[i] * (double)c->k[s * d + i];
    score *= pow(c->lam, (double)(t - s));
    for (int j = 0; j < d; ++j) o[j] += score * (double)c->v[s * d + j];
  }
  if (c->init) {
    double a = pow(c->lam, (double)(t + 1));
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) o[j] += a * (double)qt[i] * c->init[i * d + j];
  }
}

/* Output rows rows[0..n_rows) of one head, each from the decayed left
 * product directly (O(t d) per row), so single rows of very long sequences
 * can be checked.  q, k, v point at row 0 of the head ([N][d]); init is the
 * head's d x d initial state or NULL; out is [n_rows][d]. */
int oracle_rows_f64(const float *q, const float *k, const float *v, float decay, int d,
                    const int64_t *rows, int64_t n_rows, const double *init, double *out,
                    int nthreads) {
  row_ctx c = {q, k, v, (double)decay, d, rows, init, out};
  return run_units(row_unit, &c, n_rows, nthreads);
}

typedef struct {
  const float *k, *v;
  double lam;
  int d;
  int64_t N;
  const int32_t *ij;
  const double *init;
  double *out;
} ent_ctx;

static void ent_unit(void *vctx, int64_t u) {
  ent_ctx *c = (ent_ctx *)vctx;
  int d = c->d, i = c->ij[2 * u], j = c->ij[2 * u + 1];
  double acc = c->init ? pow(c->lam, (double)c->N) * c->init[i * d + j] : 0.0;
  for (int64_t s = 0; s < c->N; ++s)
    acc += pow(c->lam, (double)(c->N - 1 - s)) * (double)c->k[s * d + i] * (double)c->v[s * d + j];
  c->out[u] = acc;
}

/* Entries (i, j) of one head's state after N tokens, each as the decayed sum
 * S[i][j] = lambda^N S_init[i][j] + sum_s lambda^(N-1-s) k_s[i] v_s[j]
 * (O(N) per entry).  ij holds n pairs (i, j); out is [n]. */
int oracle_state_entries_f64(const float *k, const float *v, float decay, int d, int64_t N,
                             const int32_t *ij, int64_t n, const double *init, double *out,
                             int nthreads) {
  ent_ctx c = {k, v, (double)decay, d, N, ij, init, out};
  return run_units(ent_unit, &c, n, nthreads);
}

/* ------------------------------------------ normalisation, SiLU and gate */

/*
 * The MiniMax-01 report (section 2.2.1, before the lightning-attention
 * derivation) names normalisation, a SiLU activation and a gating mechanism
 * around the attention of its TransNormer blocks and leaves them out of the
 * derivation; the pages give no formula for any of them.  The reading
 * computed here (each part selected by a bit of `flags`):
 *
 *   bit 0, 1, 2  q', k', v' = SiLU(q), SiLU(k), SiLU(v), SiLU(x) = x / (1 + e^-x),
 *                elementwise on the inputs (else the inputs themselves);
 *   o_t          the decayed recurrence above over q', k', v';
 *   bit 3        o_t <- o_t / sqrt(mean_j o_t[j]^2 + eps) * w[h][j]: RMS
 *                normalisation over each head's d channels with a
 *                per-channel weight w [H][d] (NULL = all ones);
 *   bit 4        o_t <- o_t * sigmoid(g_t), sigmoid(x) = 1 / (1 + e^-x), with
 *                g [B][H][N][d] the gate input (an output gate).
 *
 * The final state is the recurrence's over q', k', v'.  Layout as
 * oracle_fwd_f64.
 */
#ifndef ORACLE_PLANT_GATED
#define ORACLE_PLANT_GATED 0 /* 1 = norm over tokens, not channels; 2 = gate without the
                                sigmoid; 3 = SiLU as x / (1 + e^x) (planted mistakes) */
#endif

#define ORACLE_SILU_Q 1
#define ORACLE_SILU_K 2
#define ORACLE_SILU_V 4
#define ORACLE_NORM 8
#define ORACLE_GATE 16

static double silu(double x) {
  return ORACLE_PLANT_GATED == 3 ? x / (1.0 + exp(x)) : x / (1.0 + exp(-x));
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

typedef struct {
  const float *q, *k, *v, *decay, *gate, *weight;
  double eps;
  int flags, H, d;
  int64_t N;
  const double *init;
  double *out, *fin;
} gated_ctx;

static void gated_unit(void *vctx, int64_t u) {
  gated_ctx *c = (gated_ctx *)vctx;
  int d = c->d, h = (int)(u % c->H);
  int64_t N = c->N, dd = (int64_t)d * d, base = u * N * d;
  double lam = (double)c->decay[h];
  double *S = (double *)malloc(sizeof(double) * (size_t)dd);
  double *qa = (double *)malloc(sizeof(double) * (size_t)d);
  double *ka = (double *)malloc(sizeof(double) * (size_t)d);
  double *va = (double *)malloc(sizeof(double) * (size_t)d);
  if (c->init) memcpy(S, c->init + u * dd, sizeof(double) * (size_t)dd);
  else memset(S, 0, sizeof(double) * (size_t)dd);
  for (int64_t t = 0; t < N; ++t) {
    const float *qt = c->q + base + t * d, *kt = c->k + base + t * d, *vt = c->v + base + t * d;
    for (int i = 0; i < d; ++i) {
      qa[i] = (c->flags & ORACLE_SILU_Q) ? silu((double)qt[i]) : (double)qt[i];
      ka[i] = (c->flags & ORACLE_SILU_K) ? silu((double)kt[i]) : (double)kt[i];
      va[i] = (c->flags & ORACLE_SILU_V) ? silu((double)vt[i]) : (double)vt[i];
    }
    /* S_t = lambda S_{t-1} + k'_t^T v'_t */
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) S[(int64_t)i * d + j] = lam * S[(int64_t)i * d + j] + ka[i] * va[j];
    if (!c->out) continue;
    /* o_t = q'_t S_t */
    double *o = c->out + base + t * d;
    for (int j = 0; j < d; ++j) o[j] = 0.0;
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) o[j] += qa[i] * S[(int64_t)i * d + j];
  }
  if (c->out && (c->flags & ORACLE_NORM)) {
    /* RMS over each row's d channels (the planted mistake: over each channel's
     * N tokens), all of them taken before any row is rescaled. */
    double *rms = (double *)malloc(sizeof(double) * (size_t)(ORACLE_PLANT_GATED == 1 ? d : N));
    if (ORACLE_PLANT_GATED == 1) {
      for (int j = 0; j < d; ++j) {
        double ms = 0.0;
        for (int64_t s = 0; s < N; ++s) ms += c->out[base + s * d + j] * c->out[base + s * d + j];
        rms[j] = sqrt(ms / (double)N + c->eps);
      }
    } else {
      for (int64_t t = 0; t < N; ++t) {
        const double *o = c->out + base + t * d;
        double ms = 0.0;
        for (int j = 0; j < d; ++j) ms += o[j] * o[j];
        rms[t] = sqrt(ms / (double)d + c->eps);
      }
    }
    for (int64_t t = 0; t < N; ++t) {
      double *o = c->out + base + t * d;
      for (int j = 0; j < d; ++j) {
        double w = c->weight ? (double)c->weight[(int64_t)h * d + j] : 1.0;
        o[j] = o[j] / rms[ORACLE_PLANT_GATED == 1 ? j : t] * w;
      }
    }
    free(rms);
  }
  if (c->out && (c->flags & ORACLE_GATE)) {
    for (int64_t t = 0; t < N; ++t) {
      double *o = c->out + base + t * d;
      const float *g = c->gate + base + t * d;
      for (int j = 0; j < d; ++j)
        o[j] *= ORACLE_PLANT_GATED == 2 ? (double)g[j] : sigmoid((double)g[j]);
    }
  }
  if (c->fin) memcpy(c->fin + u * dd, S, sizeof(double) * (size_t)dd);
  free(va);
  free(ka);
  free(qa);
  free(S);
}

/* The gated reading over [B][H][N][d]; gate [B][H][N][d] (needed with bit
 * 4), weight [H][d] or NULL, eps >= 0.  Returns the number of threads used. */
int oracle_fwd_gated_f64(const float *q, const float *k, const float *v, const float *decay,
                         const float *gate, const float *weight, double eps, int flags, int B,
                         int H, int64_t N, int d, const double *init, double *out, double *fin,
                         int nthreads) {
  gated_ctx c = {q, k, v, decay, gate, weight, eps, flags, H, d, N, init, out, fin};
  return run_units(gated_unit, &c, (int64_t)B * H, nthreads);
}
