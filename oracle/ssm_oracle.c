/*
 * Selective-scan oracle: the plain, slow, fp64 CPU definition.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do. It shares no code, header, table or helper with the HIP
 * library.
 *
 * What it computes (for every batch row b and channel e; n = 0..N-1):
 *   API and shapes: "scan output is different between sequential and
 *   parallel versions" (mamba.py issue 26), first reply, the API comment of
 *   the test script: x, delta (Bs, L, ED); A (ED, N); B, C (Bs, L, N);
 *   D (ED); y (Bs, L, ED). The sequential form is that page's
 *   selective_scan_seq.
 *   Recurrence (zero initial state, raw delta, Euler-style input term):
 *     a_t[n] = exp(delta[b,t,e] * A[e,n])
 *     h_t[n] = a_t[n] * h_{t-1}[n] + (delta[b,t,e] * x[b,t,e]) * B[b,t,n],  h_{-1} = 0
 *     y[b,t,e] = sum_n C[b,t,n] * h_t[n] + D[e] * x[b,t,e]
 *   Initial state: h_{-1} = 0, or h0[b,e,n] when an initial state is given
 *   (resuming a sequence from a carried state; the chunked forward of
 *   "Some questions of Bi-Mamba2 and Hydra" returns per-direction final
 *   states for exactly this use).
 *   Final state h_last[b,e,n] = h_{L-1}[n] (the forward scan's final state,
 *   as the Bi-Mamba2 forward returns per direction: "Some questions of
 *   Bi-Mamba2 and Hydra", the MambaChunkScanCombinedFn.forward listing).
 *   Bidirectional variant (same page, Hprairie's first reply, point 1 and 3:
 *   two SSMs with shared weights added together, plus D x, read in place):
 *     g_t[n] = a_t[n] * g_{t+1}[n] + (delta x)[t] * B[b,t,n],  g_L = 0
 *     y[b,t,e] = sum_n C[b,t,n] * (h_t[n] + g_t[n]) + D[e] * x[b,t,e]
 *   with the same a_t, inputs read in place (no shift, no flipped copy).
 *   The reverse state may also enter from a carried state, g_L = g0[b,e,n]
 *   (the reverse direction's counterpart of h0: the Bi-Mamba2 forward
 *   returns a final state per direction, final_states_f and final_states_b,
 *   and a sequence cut in two resumes each direction from the other piece's).
 *
 * Optional step-size pre-processing and output gate, the options of the
 * Bi-Mamba2 forward (same page, the MambaChunkScanCombinedFn.forward
 * listing: dt_bias, dt_softplus, dt_limit, z), with their usual meaning:
 *     delta' = clamp(softplus?(delta + dt_bias[e]), dt_min, dt_max)
 *     softplus(v) = v for v > 20, else log(1 + exp(v))
 *     y' = y * z * sigmoid(z)            (z of the same shape as y)
 * delta' replaces delta everywhere above; the gate multiplies the complete
 * output (both directions and the D x term).
 *
 * Backward pass (oracle_scan_bwd): the gradients of sum(dy * y) for the
 * forward scan without options, the step the Bi-Mamba2 page's autograd
 * function takes after the forward ("Some questions of Bi-Mamba2 and Hydra",
 * the backward listing: dx, ddt, dA, dB, dC, dD from dout). The pages give
 * no formula; it is the adjoint of the recurrence above, derived by the chain
 * rule and written out where the function is defined.
 *
 * Every product of two fp32 (or bf16) inputs is exact in fp64; exp is the
 * host libm's. Threads split only the independent (b, e) channels; the
 * arithmetic of each channel runs in the order written above.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

static double load(const void* p, int64_t i, int dtype) {
  if (dtype == ORACLE_BF16) {
    uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
  }
  return (double)((const float*)p)[i];
}

struct work;
static double step_size(const struct work* w, int64_t ix, int64_t e);

typedef struct work {
  int dtype, bidir;
  const void *x, *delta, *B, *C;
  const float *A, *D;
  const float* h0; /* (Bs, ED, N) initial forward state, or NULL for zero */
  const float* g0; /* (Bs, ED, N) reverse state entering at t = L-1 (bidir), or NULL for zero */
  const float* dt_bias; /* (ED) or NULL */
  int dt_softplus;
  double dt_min, dt_max;
  const void* z;   /* (Bs, L, ED) gate, same dtype as x, or NULL */
  int64_t Bs, L, ED, N;
  const int64_t* chans; /* channel ids c = b*ED + e, or NULL for all */
  int64_t nchans;
  double* y;      /* (nchans, L): y of channel k at row k */
  double* h_last; /* (nchans, N) or NULL */
  double* g_first;/* (nchans, N) or NULL: reverse state at t = 0 (bidir only) */
  int64_t k0, k1; /* this worker's range of k */
} work_t;

/* clamp(softplus?(v + bias), dt_min, dt_max); bias is dt_bias[e] or 0 */
static double step_map(double v, double bias, int softplus, double dt_min, double dt_max) {
  v += bias;
  if (softplus) v = v > 20.0 ? v : log1p(exp(v));
  if (v < dt_min) v = dt_min;
  if (v > dt_max) v = dt_max;
  return v;
}

/* d delta' / d delta of step_map at v (the derivative of the clamp is taken
   as 0 at and beyond its bounds, 1 inside; softplus' = sigmoid below 20, 1
   above, matching the map) */
static double step_map_deriv(double v, double bias, int softplus, double dt_min, double dt_max) {
  v += bias;
  double u = v, d = 1.0;
  if (softplus && v <= 20.0) {
    u = log1p(exp(v));
    d = 1.0 / (1.0 + exp(-v));
  }
  if (u <= dt_min || u >= dt_max) d = 0.0;
  return d;
}

/* delta' for the element at index ix of channel e */
static double step_size(const struct work* w, int64_t ix, int64_t e) {
  return step_map(load(w->delta, ix, w->dtype), w->dt_bias ? (double)w->dt_bias[e] : 0.0, w->dt_softplus,
                  w->dt_min, w->dt_max);
}

/* One channel: the forward recurrence, then (bidir) the reverse one. */
static void scan_channel(const work_t* w, int64_t k, double* h, double* g) {
  const int64_t c = w->chans ? w->chans[k] : k;
  const int64_t b = c / w->ED, e = c % w->ED;
  const int64_t L = w->L, ED = w->ED, N = w->N;
  double* y = w->y + k * L;

  for (int64_t n = 0; n < N; ++n) h[n] = w->h0 ? (double)w->h0[(b * ED + e) * N + n] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const int64_t ix = (b * L + t) * ED + e; /* x, delta index */
    const int64_t ib = (b * L + t) * N;      /* B, C row index */
    const double dt = step_size(w, ix, e);
    const double xv = load(w->x, ix, w->dtype);
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double a = exp(dt * (double)w->A[e * N + n]);
      h[n] = a * h[n] + (dt * xv) * load(w->B, ib + n, w->dtype);
      acc += load(w->C, ib + n, w->dtype) * h[n];
    }
    y[t] = acc;
  }
  if (w->h_last)
    for (int64_t n = 0; n < N; ++n) w->h_last[k * N + n] = h[n];

  if (w->bidir) {
    for (int64_t n = 0; n < N; ++n) g[n] = w->g0 ? (double)w->g0[(b * ED + e) * N + n] : 0.0;
    for (int64_t t = L - 1; t >= 0; --t) {
      const int64_t ix = (b * L + t) * ED + e;
      const int64_t ib = (b * L + t) * N;
      const double dt = step_size(w, ix, e);
      const double xv = load(w->x, ix, w->dtype);
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        const double a = exp(dt * (double)w->A[e * N + n]);
        g[n] = a * g[n] + (dt * xv) * load(w->B, ib + n, w->dtype);
        acc += load(w->C, ib + n, w->dtype) * g[n];
      }
      y[t] += acc;
    }
    if (w->g_first)
      for (int64_t n = 0; n < N; ++n) w->g_first[k * N + n] = g[n];
  }

  /* the skip term D x, added once; then the gate */
  for (int64_t t = 0; t < L; ++t) {
    const int64_t ix = (b * L + t) * ED + e;
    const double xv = load(w->x, ix, w->dtype);
    const double d = w->D ? (double)w->D[e] : 0.0;
    y[t] += d * xv;
    if (w->z) {
      const double zv = load(w->z, ix, w->dtype);
      y[t] *= zv / (1.0 + exp(-zv));
    }
  }
}

static void* worker(void* p) {
  work_t* w = (work_t*)p;
  double* h = (double*)malloc(sizeof(double) * (size_t)w->N * 2);
  if (!h) return (void*)1;
  for (int64_t k = w->k0; k < w->k1; ++k) scan_channel(w, k, h, h + w->N);
  free(h);
  return NULL;
}

/*
 * Run the oracle over the listed channels (or all Bs*ED channels when chans
 * is NULL, in order c = b*ED + e). Outputs are channel-major:
 * y[k*L + t], h_last[k*N + n], g_first[k*N + n]. Returns 0 on success,
 * -1 on bad arguments, -2 when memory for a worker could not be allocated.
 */
int oracle_scan(int dtype, int bidir, const void* x, const void* delta, const float* A, const void* B,
                const void* C, const float* D, const float* h0, const float* g0, const float* dt_bias, int dt_softplus,
                double dt_min, double dt_max, const void* z, int64_t Bs, int64_t L, int64_t ED, int64_t N,
                const int64_t* chans, int64_t nchans, double* y, double* h_last, double* g_first,
                int nthreads) {
  if (!x || !delta || !A || !B || !C || !y) return -1;
  /* empty batches, sequences or channel sets are allowed: over zero steps the
     state stays where it entered (h0, or zero) */
  if (Bs < 0 || L < 0 || ED < 0 || N <= 0) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  if (!chans) nchans = Bs * ED;
  if (nchans < 0) return -1;
  for (int64_t k = 0; chans && k < nchans; ++k)
    if (chans[k] < 0 || chans[k] >= Bs * ED) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > nchans) nthreads = (int)(nchans > 0 ? nchans : 1);

  work_t base = {dtype, bidir, x, delta, B, C, A, D, h0, bidir ? g0 : NULL, dt_bias, dt_softplus, dt_min, dt_max, z,
                 Bs, L, ED, N, chans, nchans, y, h_last,
                 bidir ? g_first : NULL, 0, 0};
  work_t* ws = (work_t*)malloc(sizeof(work_t) * (size_t)nthreads);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!ws || !th) {
    free(ws);
    free(th);
    return -2;
  }
  int64_t per = (nchans + nthreads - 1) / nthreads;
  for (int i = 0; i < nthreads; ++i) {
    ws[i] = base;
    ws[i].k0 = per * i < nchans ? per * i : nchans;
    ws[i].k1 = per * (i + 1) < nchans ? per * (i + 1) : nchans;
  }
  int rc = 0;
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &ws[i]);
  if (worker(&ws[0])) rc = -2;
  for (int i = 1; i < nthreads; ++i) {
    void* r = NULL;
    pthread_join(th[i], &r);
    if (r) rc = -2;
  }
  free(ws);
  free(th);
  return rc;
}

/*
 * Backward pass of the forward scan (the bidirectional variant is composed
 * from it in oracle/__init__.py): given dy = dL/dy, the gradients of L with
 * respect to every input, by the adjoint of the recurrence above, where
 * delta_t stands for the mapped step size delta' of the options and dy_t for
 * the scan's own output gradient, dy z sigmoid(z) under a gate (the gate's
 * dz needs the whole output and is formed by the Python wrapper). The raw
 * step size gets ddelta times d delta'/d delta (step_map_deriv), and
 * ddt_bias[e] is the sum over (b, t) of that. With g_t[n] = dL/dh_t[n]:
 *     g_t = dy_t C_t + a_{t+1} g_{t+1}          (reverse time; a_L g_L = dh_last)
 *     dC[b,t,n] = sum_e dy_t h_t[n]             dD[e] = sum_{b,t} dy_t x_t
 *     dx_t = sum_n g_t[n] delta_t B_t[n] + dy_t D[e]
 *     ddelta_t = sum_n g_t[n] (x_t B_t[n] + A[e,n] a_t[n] h_{t-1}[n])
 *     dB[b,t,n] = sum_e g_t[n] delta_t x_t
 *     dA[e,n] = sum_{b,t} g_t[n] a_t[n] h_{t-1}[n] delta_t
 *     dh0 = a_0 g_0 (h_{-1} = h0)
 * Rows are done one after the other; the channels of a row are cut into
 * fixed blocks of 64 that threads share. dB and dC of a row are the sums of
 * the blocks' partial sums in block order, and dA and dD the sums of the
 * rows' in row order, so the result does not depend on the thread count. Outputs are fp64:
 * dx, ddelta (Bs, L, ED); dA (ED, N); dB, dC (Bs, L, N); dD (ED);
 * dh0 (Bs, ED, N) or NULL; ddt_bias (ED) or NULL. y is affine in h0, so dh0 does not depend on h0
 * and is returned for h0 = NULL (the zero initial state) as well.
 * dh_last (Bs, ED, N), or NULL for zero, is the gradient of the loss with
 * respect to the final state h_{L-1} (the backward listing of the Bi-Mamba2
 * page takes it as dfinal_states): the loss is sum(dy * y) + sum(dh_last *
 * h_{L-1}), so the adjoint enters the last step with g_{L-1} = dy C + dh_last.
 */
enum { BWD_BLOCK = 64 }; /* channels per work item */

typedef struct {
  int dtype;
  const void *x, *delta, *B, *C, *dy;
  const float *A, *D, *h0;
  const float* dh_last; /* (Bs, ED, N) gradient of the final state, or NULL */
  const float* dt_bias; /* (ED) or NULL */
  int dt_softplus;
  double dt_min, dt_max;
  const void* z;        /* gate (Bs, L, ED) or NULL: dy is taken as dy z sigmoid(z) */
  int64_t Bs, L, ED, N;
  double *dx, *ddelta, *dh0;
  double *dA_part, *dD_part, *dbias_part; /* per row: (Bs, ED, N), (Bs, ED), (Bs, ED) */
  double *partB, *partC;     /* per channel block of the current row: (nblk, L, N) */
  int64_t b, blk0, blk1;     /* row, channel blocks [blk0, blk1) */
  int fail;
} bwd_t;

static void* bwd_worker(void* p) {
  bwd_t* w = (bwd_t*)p;
  const int64_t L = w->L, ED = w->ED, N = w->N, b = w->b;
  double* hs = (double*)malloc(sizeof(double) * (size_t)(L + 1) * N); /* h_{t-1} at row t */
  double* g = (double*)malloc(sizeof(double) * (size_t)N);
  if (!hs || !g) {
    free(hs);
    free(g);
    w->fail = 1;
    return NULL;
  }
  for (int64_t blk = w->blk0; blk < w->blk1; ++blk) {
    double* pB = w->partB + blk * L * N;
    double* pC = w->partC + blk * L * N;
    for (int64_t i = 0; i < L * N; ++i) pB[i] = 0.0, pC[i] = 0.0;
    const int64_t e1 = (blk + 1) * BWD_BLOCK < ED ? (blk + 1) * BWD_BLOCK : ED;
    for (int64_t e = blk * BWD_BLOCK; e < e1; ++e) {
      const double bias = w->dt_bias ? (double)w->dt_bias[e] : 0.0;
      /* forward, keeping every state */
      for (int64_t n = 0; n < N; ++n) hs[n] = w->h0 ? (double)w->h0[(b * ED + e) * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        const int64_t ix = (b * L + t) * ED + e, ib = (b * L + t) * N;
        const double dt = step_map(load(w->delta, ix, w->dtype), bias, w->dt_softplus, w->dt_min, w->dt_max);
        const double xv = load(w->x, ix, w->dtype);
        for (int64_t n = 0; n < N; ++n) {
          const double a = exp(dt * (double)w->A[e * N + n]);
          hs[(t + 1) * N + n] = a * hs[t * N + n] + (dt * xv) * load(w->B, ib + n, w->dtype);
        }
      }
      /* reverse: the adjoint state and every gradient term; g holds a_{t+1}
         g_{t+1} at the top of step t, which at t = L-1 is the final state's
         own gradient */
      for (int64_t n = 0; n < N; ++n) g[n] = w->dh_last ? (double)w->dh_last[(b * ED + e) * N + n] : 0.0;
      double dD = 0.0;
      double* dA = w->dA_part + (b * ED + e) * N;
      for (int64_t n = 0; n < N; ++n) dA[n] = 0.0;
      double dbias = 0.0;
      for (int64_t t = L - 1; t >= 0; --t) {
        const int64_t ix = (b * L + t) * ED + e, ib = (b * L + t) * N;
        const double raw = load(w->delta, ix, w->dtype);
        const double dt = step_map(raw, bias, w->dt_softplus, w->dt_min, w->dt_max);
        const double xv = load(w->x, ix, w->dtype);
        double dyv = load(w->dy, ix, w->dtype);
        if (w->z) { /* the scan's output is gated: its own output gradient is dy z sigmoid(z) */
          const double zv = load(w->z, ix, w->dtype);
          dyv *= zv / (1.0 + exp(-zv));
        }
        double dxv = w->D ? dyv * (double)w->D[e] : 0.0, ddv = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double An = (double)w->A[e * N + n];
          const double Bv = load(w->B, ib + n, w->dtype), Cv = load(w->C, ib + n, w->dtype);
          /* g_t = dy_t C_t + a_{t+1} g_{t+1}: g[n] holds a_{t+1} g_{t+1} here */
          g[n] += dyv * Cv;
          const double a = exp(dt * An);
          const double hprev = hs[t * N + n];
          pC[t * N + n] += dyv * hs[(t + 1) * N + n];
          pB[t * N + n] += g[n] * dt * xv;
          dxv += g[n] * dt * Bv;
          ddv += g[n] * (xv * Bv + An * a * hprev);
          dA[n] += g[n] * a * hprev * dt;
          g[n] *= a; /* a_t g_t, the carry into step t-1 */
        }
        dD += dyv * xv;
        w->dx[ix] = dxv;
        /* through the step-size map: d/d(raw delta) = d/d(delta') * delta'(raw) */
        const double ddr = ddv * step_map_deriv(raw, bias, w->dt_softplus, w->dt_min, w->dt_max);
        w->ddelta[ix] = ddr;
        dbias += ddr;
      }
      if (w->dh0)
        for (int64_t n = 0; n < N; ++n) w->dh0[(b * ED + e) * N + n] = g[n];
      w->dD_part[b * ED + e] = dD;
      w->dbias_part[b * ED + e] = dbias;
    }
  }
  free(hs);
  free(g);
  return NULL;
}

int oracle_scan_bwd(int dtype, const void* x, const void* delta, const float* A, const void* B, const void* C,
                    const float* D, const float* h0, const float* dh_last, const float* dt_bias, int dt_softplus,
                    double dt_min,
                    double dt_max, const void* z, const void* dy, int64_t Bs, int64_t L, int64_t ED, int64_t N,
                    double* dx, double* ddelta, double* dA, double* dB, double* dC, double* dD, double* dh0,
                    double* ddt_bias, int nthreads) {
  if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB || !dC || !dD) return -1;
  if (Bs < 0 || L < 0 || ED < 0 || N <= 0) return -1; /* empty sizes allowed */
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  const int64_t nblk = (ED + BWD_BLOCK - 1) / BWD_BLOCK;
  if (nthreads > nblk) nthreads = (int)nblk;
  if (nthreads > 256) nthreads = 256;
  if (nthreads < 1) nthreads = 1;
  /* (one element more than needed, so that empty sizes still get a buffer) */
  double* dA_part = (double*)malloc(sizeof(double) * (size_t)(Bs * ED * N + 1));
  double* dD_part = (double*)malloc(sizeof(double) * (size_t)(Bs * ED + 1));
  double* dbias_part = (double*)malloc(sizeof(double) * (size_t)(Bs * ED + 1));
  double* partB = (double*)malloc(sizeof(double) * (size_t)(nblk * L * N + 1));
  double* partC = (double*)malloc(sizeof(double) * (size_t)(nblk * L * N + 1));
  bwd_t* ws = (bwd_t*)malloc(sizeof(bwd_t) * (size_t)nthreads);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  int rc = 0;
  if (!dA_part || !dD_part || !dbias_part || !partB || !partC || !ws || !th) rc = -2;
  /* one batch row at a time; its channel blocks are split over the threads,
     and dB, dC of the row are the sums of the blocks' partials in block order */
  for (int64_t b = 0; rc == 0 && b < Bs; ++b) {
    const int64_t per = (nblk + nthreads - 1) / nthreads;
    for (int i = 0; i < nthreads; ++i) {
      ws[i] = (bwd_t){dtype, x, delta, B, C, dy, A, D, h0, dh_last, dt_bias, dt_softplus, dt_min, dt_max, z,
                      Bs, L, ED, N, dx, ddelta, dh0, dA_part, dD_part, dbias_part, partB, partC, b, 0, 0, 0};
      ws[i].blk0 = per * i < nblk ? per * i : nblk;
      ws[i].blk1 = per * (i + 1) < nblk ? per * (i + 1) : nblk;
    }
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, bwd_worker, &ws[i]);
    bwd_worker(&ws[0]);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; ++i)
      if (ws[i].fail) rc = -2;
    for (int64_t i = 0; rc == 0 && i < L * N; ++i) {
      double sb = 0.0, sc = 0.0;
      for (int64_t k = 0; k < nblk; ++k) sb += partB[k * L * N + i], sc += partC[k * L * N + i];
      dB[b * L * N + i] = sb;
      dC[b * L * N + i] = sc;
    }
  }
  /* sums over batch rows, in row order */
  for (int64_t i = 0; rc == 0 && i < ED * N; ++i) {
    double s = 0.0;
    for (int64_t b = 0; b < Bs; ++b) s += dA_part[b * ED * N + i];
    dA[i] = s;
  }
  for (int64_t e = 0; rc == 0 && e < ED; ++e) {
    double s = 0.0;
    for (int64_t b = 0; b < Bs; ++b) s += dD_part[b * ED + e];
    dD[e] = s;
  }
  for (int64_t e = 0; rc == 0 && ddt_bias && e < ED; ++e) {
    double s = 0.0;
    for (int64_t b = 0; b < Bs; ++b) s += dbias_part[b * ED + e];
    ddt_bias[e] = s;
  }
  free(dA_part);
  free(dD_part);
  free(dbias_part);
  free(partB);
  free(partC);
  free(ws);
  free(th);
  return rc;
}

/*
 * Multi-head (Mamba-2 / SSD) selective scan, the layout of the chunked scan
 * the Bi-Mamba2 page calls ("Some questions of Bi-Mamba2 and Hydra", the
 * MambaChunkScanCombinedFn listings): x (Bs, L, H, P), dt (Bs, L, H), a scalar
 * A per head, B and C (Bs, L, G, N) shared by the H / G heads of a group,
 * D (H). For batch row b, head h (group g = h / (H / G)), head channel p and
 * state n the recurrence is the one above with one decay per head:
 *   a_t = exp(dt[b,t,h] A[h])
 *   S_t[p][n] = a_t S_{t-1}[p][n] + (dt[b,t,h] x[b,t,h,p]) B[b,t,g,n],  S_{-1} = h0 (or 0)
 *   y[b,t,h,p] = sum_n C[b,t,g,n] S_t[p][n] + D[h] x[b,t,h,p]
 * bidir adds the reverse-time scan with the same a_t (no shift, D x once):
 *   R_t = a_t R_{t+1} + (dt x)_t B_t,  R_L = g0 (or 0),   y += sum_n C_t R_t.
 * The same options as the per-channel form, with the head in place of the
 * channel (the forward listing of the Bi-Mamba2 page passes dt_bias per head
 * and z of x's shape to this scan):
 *   dt' = clamp(softplus?(dt[b,t,h] + dt_bias[h]), dt_min, dt_max) replaces dt,
 *   y'[b,t,h,p] = y[b,t,h,p] z sigmoid(z), z = z[b,t,h,p] (the complete output).
 * The chunk length of the pages' kernels does not change the result; this
 * definition has none. Outputs fp64: y (Bs, L, H, P); h_last and g_first
 * (Bs, H, P, N) or NULL. Threads split the independent (b, h) pairs.
 */
typedef struct {
  int dtype, bidir;
  const void *x, *dt, *B, *C;
  const float *A, *D, *h0;
  const float* g0;      /* (Bs, H, P, N) reverse state entering at t = L-1, or NULL */
  const float* dt_bias; /* (H) or NULL */
  int dt_softplus;
  double dt_min, dt_max;
  const void* z; /* (Bs, L, H, P) gate, x's dtype, or NULL */
  int64_t Bs, L, H, P, G, N;
  double *y, *h_last, *g_first;
  int64_t k0, k1; /* (b, h) pairs [k0, k1) */
  int fail;
} ssd_t;

static void* ssd_worker(void* arg) {
  ssd_t* w = (ssd_t*)arg;
  const int64_t L = w->L, H = w->H, P = w->P, G = w->G, N = w->N;
  double* S = (double*)malloc(sizeof(double) * (size_t)(P * N));
  if (!S) {
    w->fail = 1;
    return NULL;
  }
  for (int64_t k = w->k0; k < w->k1; ++k) {
    const int64_t b = k / H, h = k % H, g = h / (H / G);
    const double Ah = (double)w->A[h];
    const double Dh = w->D ? (double)w->D[h] : 0.0;
    for (int dir = 0; dir < (w->bidir ? 2 : 1); ++dir) {
      const float* init = dir == 0 ? w->h0 : w->g0;
      for (int64_t i = 0; i < P * N; ++i) S[i] = init ? (double)init[(b * H + h) * P * N + i] : 0.0;
      for (int64_t s = 0; s < L; ++s) {
        const int64_t t = dir == 0 ? s : L - 1 - s;
        const double dtv = step_map(load(w->dt, (b * L + t) * H + h, w->dtype),
                                    w->dt_bias ? (double)w->dt_bias[h] : 0.0, w->dt_softplus, w->dt_min, w->dt_max);
        const double a = exp(dtv * Ah);
        const int64_t ib = ((b * L + t) * G + g) * N;
        for (int64_t p = 0; p < P; ++p) {
          const int64_t ix = ((b * L + t) * H + h) * P + p;
          const double xv = load(w->x, ix, w->dtype);
          double acc = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            S[p * N + n] = a * S[p * N + n] + (dtv * xv) * load(w->B, ib + n, w->dtype);
            acc += load(w->C, ib + n, w->dtype) * S[p * N + n];
          }
          if (dir == 0)
            w->y[ix] = acc + Dh * xv;
          else
            w->y[ix] += acc;
        }
      }
      double* out = dir == 0 ? w->h_last : w->g_first;
      if (out)
        for (int64_t i = 0; i < P * N; ++i) out[(b * H + h) * P * N + i] = S[i];
    }
    /* the gate multiplies the complete output of the head */
    if (w->z)
      for (int64_t t = 0; t < L; ++t)
        for (int64_t p = 0; p < P; ++p) {
          const int64_t ix = ((b * L + t) * H + h) * P + p;
          const double zv = load(w->z, ix, w->dtype);
          w->y[ix] *= zv / (1.0 + exp(-zv));
        }
  }
  free(S);
  return NULL;
}

int oracle_ssd(int dtype, int bidir, const void* x, const void* dt, const float* A, const void* B, const void* C,
               const float* D, const float* h0, const float* g0, const float* dt_bias, int dt_softplus, double dt_min, double dt_max,
               const void* z, int64_t Bs, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, double* y,
               double* h_last, double* g_first, int nthreads) {
  if (!x || !dt || !A || !B || !C || !y) return -1;
  /* empty batches or sequences are allowed (over zero steps the state stays h0) */
  if (Bs < 0 || L < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G != 0) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  const int64_t K = Bs * H;
  if (nthreads > K) nthreads = (int)K;
  if (nthreads > 256) nthreads = 256;
  if (nthreads < 1) nthreads = 1;
  ssd_t* ws = (ssd_t*)malloc(sizeof(ssd_t) * (size_t)nthreads);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!ws || !th) {
    free(ws);
    free(th);
    return -2;
  }
  const int64_t per = (K + nthreads - 1) / nthreads;
  for (int i = 0; i < nthreads; ++i) {
    ws[i] = (ssd_t){dtype, bidir, x, dt, B, C, A, D, h0, bidir ? g0 : NULL, dt_bias, dt_softplus, dt_min, dt_max, z,
                    Bs, L, H, P, G, N, y, h_last, bidir ? g_first : NULL, 0, 0, 0};
    ws[i].k0 = per * i < K ? per * i : K;
    ws[i].k1 = per * (i + 1) < K ? per * (i + 1) : K;
  }
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, ssd_worker, &ws[i]);
  ssd_worker(&ws[0]);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
  int rc = 0;
  for (int i = 0; i < nthreads; ++i)
    if (ws[i].fail) rc = -2;
  free(ws);
  free(th);
  return rc;
}
