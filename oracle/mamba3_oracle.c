/*
 * Mamba-3 SSM layer core -- plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or run this code.  It shares nothing
 * with the HIP path (no headers, helpers, tables or constants) and never
 * imports it.
 *
 * What it computes (the pages are cited by title and section):
 *
 *   linkstar.cloud/article/869, section "第一刀：指数梯形离散化" (exponential-
 *   trapezoidal discretisation): with alpha_t = exp(dt_t A_t),
 *   beta_t = (1 - lam_t) dt_t alpha_t and gamma_t = lam_t dt_t the state obeys
 *       h_t = alpha_t h_{t-1} + beta_t B_{t-1} x_{t-1}^T + gamma_t B_t x_t^T.
 *
 *   same page, section "第二刀：复值状态空间" (complex-valued state and the
 *   RoPE trick): the complex state is a real state of twice the size whose
 *   transition holds 2x2 rotations R(theta) = [[cos,-sin],[sin,cos]] built from
 *   dt_t theta_t, and those rotations can be moved onto B and C as cumulative
 *   (data-dependent) rotary angles.
 *
 *   same page, section "第三刀：多输入多输出" (MIMO): B_t is N x R and x_t is
 *   P x R, so the input term is the rank-R product B_t x_t^T; the output is
 *   y_t = C_t^T h_t (R x P).
 *
 * The recurrence is evaluated token by token, in the rotated (RoPE) frame, in
 * double precision, exactly as those three passages combine:
 *
 *   phi_t[k]   = sum_{s<=t} dt_s theta_s[k]          (inclusive of t)
 *   Bt_t, Ct_t = R(-phi_t) applied to each pair (2k, 2k+1) of every rank
 *   ht_t       = alpha_t ht_{t-1} + beta_t sum_r Bt_{t-1}[r] x_{t-1}[r]^T
 *                                 + gamma_t sum_r Bt_t[r] x_t[r]^T
 *   y_t[r]     = Ct_t[r]^T ht_t
 *   h_final    = R(+phi_L) ht_L    (back to the un-rotated, "true" frame)
 *
 * Readings where the pages are silent:
 *  - the token before the first one (prev_B, prev_x) sits at angle 0, i.e.
 *    in the starting frame; absent, it is zero;
 *  - h0 is given in the true frame, which equals the rotated frame at angle 0;
 *  - the final state carries no pending trapezoid term (nothing after t = L);
 *  - B and C pair (2k, 2k+1) = (real, imaginary) of complex component k.
 *
 * Layouts (row-major, contiguous):
 *   x, y (B,L,H,R,P); Bm, Cm (B,L,H,R,N); dt, A, lam (B,L,H);
 *   theta (B,L,H,N/2); h0, h_final (B,H,N,P); prev_B (B,H,R,N);
 *   prev_x (B,H,R,P); angle0, angle_final (B,H,N/2).
 *
 * Parity is pinned by tests/test_oracle_pins.py (literal complex arithmetic,
 * the lambda = 1 and theta = 0 special cases, a hand-set parity sequence,
 * scalar closed forms, the convergence order, MIMO superposition and the
 * quadratic "1-semiseparable x 2-band" form), none of which call this code's
 * formulas.
 *
 * The backward (gradients of a linear functional of y and h_final) is the
 * chain rule of this same computation in reverse order; it is pinned against
 * central finite differences of the forward.
 *
 * Compile-time switch ORACLE_MUTANT (tests only): plants one known mistake so
 * that a test can show that the pins catch it.  Never set in a normal build.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

typedef struct {
  int64_t B, L, H, P, N, R;
  const double *x, *Bm, *Cm, *dt, *A, *lam, *theta, *h0, *prev_B, *prev_x;
  double *y, *h_final;
  int64_t slice_begin, slice_end;
  int status;
} fwd_job;

/* rotate pair (u, v) by angle a: R(a) (u, v) = (u cos a - v sin a, u sin a + v cos a) */
static void rot(double a, double u, double v, double* ou, double* ov) {
  double c = cos(a), s = sin(a);
  *ou = c * u - s * v;
  *ov = s * u + c * v;
}

static void fwd_slice(const fwd_job* j, int64_t bh) {
  const int64_t B = j->B, L = j->L, H = j->H, P = j->P, N = j->N, R = j->R;
  const int64_t K = N / 2;
  const int64_t b = bh / H, h = bh % H;
  (void)B;
  double* hs = (double*)calloc((size_t)(N * P), sizeof(double));
  double* phi = (double*)calloc((size_t)K, sizeof(double));
  double* Bprev = (double*)calloc((size_t)(R * N), sizeof(double));
  double* xprev = (double*)calloc((size_t)(R * P), sizeof(double));
  double* Bcur = (double*)malloc(sizeof(double) * (size_t)(R * N));
  double* Ccur = (double*)malloc(sizeof(double) * (size_t)(R * N));
  const double* xcur;

  if (j->h0) memcpy(hs, j->h0 + bh * N * P, sizeof(double) * (size_t)(N * P));
#if ORACLE_MUTANT == 8
  if (0) { /* mutant: the token before the first one is ignored */
#else
  if (j->prev_B && j->prev_x) {
#endif
    /* the previous token sits at angle 0: its rotated B equals its raw B */
    memcpy(Bprev, j->prev_B + bh * R * N, sizeof(double) * (size_t)(R * N));
    memcpy(xprev, j->prev_x + bh * R * P, sizeof(double) * (size_t)(R * P));
  }

  for (int64_t t = 0; t < L; ++t) {
    const int64_t tok = (b * L + t) * H + h; /* index into (B,L,H) */
    const double dt = j->dt[tok], A = j->A[tok], lam = j->lam[tok];
    const double* th = j->theta + tok * K;
    const double* Braw = j->Bm + tok * R * N;
    const double* Craw = j->Cm + tok * R * N;
    xcur = j->x + tok * R * P;

    /* cumulative angle, inclusive of this token */
    for (int64_t k = 0; k < K; ++k) phi[k] += dt * th[k];
    /* B~ = R(-phi) B, C~ = R(-phi) C on every pair of every rank */
    for (int64_t r = 0; r < R; ++r)
      for (int64_t k = 0; k < K; ++k) {
        double a = -phi[k];
#if ORACLE_MUTANT == 2
        a = phi[k]; /* mutant: wrong rotation sign */
#endif
#if ORACLE_MUTANT == 3
        a = -(phi[k] - dt * th[k]); /* mutant: exclusive angle (lags one token) */
#endif
        rot(a, Braw[r * N + 2 * k], Braw[r * N + 2 * k + 1], &Bcur[r * N + 2 * k], &Bcur[r * N + 2 * k + 1]);
        rot(a, Craw[r * N + 2 * k], Craw[r * N + 2 * k + 1], &Ccur[r * N + 2 * k], &Ccur[r * N + 2 * k + 1]);
      }

    const double alpha = exp(dt * A);
    double beta = (1.0 - lam) * dt * alpha;
    double gamma = lam * dt;
#if ORACLE_MUTANT == 1
    beta = (1.0 - lam) * dt; /* mutant: alpha dropped from beta */
#endif
#if ORACLE_MUTANT == 5
    { double tmp = beta; beta = gamma; gamma = tmp; } /* mutant: weights swapped */
#endif

    double* yt = j->y + tok * R * P;
#if ORACLE_MUTANT == 9
    for (int64_t r = 0; r < R; ++r) /* mutant: y from the state before the update */
      for (int64_t p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += Ccur[r * N + n] * hs[n * P + p];
        yt[r * P + p] = acc;
      }
#endif
    for (int64_t n = 0; n < N; ++n)
      for (int64_t p = 0; p < P; ++p) {
        double acc_prev = 0.0, acc_cur = 0.0;
        for (int64_t r = 0; r < R; ++r) {
#if ORACLE_MUTANT == 4
          acc_prev += Bcur[r * N + n] * xprev[r * P + p]; /* mutant: beta term uses B_t */
#else
          acc_prev += Bprev[r * N + n] * xprev[r * P + p];
#endif
#if ORACLE_MUTANT == 7
          if (r > 0) continue; /* mutant: only rank 0 enters the state */
#endif
          acc_cur += Bcur[r * N + n] * xcur[r * P + p];
        }
        hs[n * P + p] = alpha * hs[n * P + p] + beta * acc_prev + gamma * acc_cur;
      }

#if ORACLE_MUTANT != 9
    for (int64_t r = 0; r < R; ++r)
      for (int64_t p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += Ccur[r * N + n] * hs[n * P + p];
        yt[r * P + p] = acc;
      }
#endif

    memcpy(Bprev, Bcur, sizeof(double) * (size_t)(R * N));
    memcpy(xprev, xcur, sizeof(double) * (size_t)(R * P));
  }

  if (j->h_final) {
    double* hf = j->h_final + bh * N * P;
    for (int64_t k = 0; k < K; ++k)
      for (int64_t p = 0; p < P; ++p) {
        double u = hs[(2 * k) * P + p], v = hs[(2 * k + 1) * P + p];
#if ORACLE_MUTANT == 6
        hf[(2 * k) * P + p] = u; /* mutant: final state left in the rotated frame */
        hf[(2 * k + 1) * P + p] = v;
#else
        rot(phi[k], u, v, &hf[(2 * k) * P + p], &hf[(2 * k + 1) * P + p]);
#endif
      }
  }
  free(hs); free(phi); free(Bprev); free(xprev); free(Bcur); free(Ccur);
}

static void* fwd_worker(void* arg) {
  fwd_job* j = (fwd_job*)arg;
  for (int64_t bh = j->slice_begin; bh < j->slice_end; ++bh) fwd_slice(j, bh);
  return NULL;
}

static int pick_threads(int nthreads, int64_t work) {
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > work) nthreads = (int)work;
  if (nthreads < 1) nthreads = 1;
  return nthreads;
}

/* Returns 0 on success, -1 on bad arguments.  Every (b,h) slice is an
 * independent recurrence; slices are split statically over threads. */
int mamba3_oracle_forward(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t R,
                          const double* x, const double* Bm, const double* Cm,
                          const double* dt, const double* A, const double* lam, const double* theta,
                          const double* h0, const double* prev_B, const double* prev_x,
                          double* y, double* h_final, int nthreads) {
  if (B <= 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || R <= 0 || (N % 2) != 0) return -1;
  if (L > 0 && (!x || !Bm || !Cm || !dt || !A || !lam || !theta || !y)) return -1;
  const int64_t slices = B * H;
  const int nt = pick_threads(nthreads, slices);
  fwd_job* jobs = (fwd_job*)calloc((size_t)nt, sizeof(fwd_job));
  pthread_t* tids = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
  for (int i = 0; i < nt; ++i) {
    fwd_job* j = &jobs[i];
    j->B = B; j->L = L; j->H = H; j->P = P; j->N = N; j->R = R;
    j->x = x; j->Bm = Bm; j->Cm = Cm; j->dt = dt; j->A = A; j->lam = lam; j->theta = theta;
    j->h0 = h0; j->prev_B = prev_B; j->prev_x = prev_x; j->y = y; j->h_final = h_final;
    j->slice_begin = slices * i / nt;
    j->slice_end = slices * (i + 1) / nt;
  }
  for (int i = 1; i < nt; ++i) pthread_create(&tids[i], NULL, fwd_worker, &jobs[i]);
  fwd_worker(&jobs[0]);
  for (int i = 1; i < nt; ++i) pthread_join(tids[i], NULL);
  free(jobs); free(tids);
  return 0;
}

/* ------------------------------------------------------------------------
 * Backward (reverse mode) of the forward above.
 *
 * The gradient of the scalar  l = sum_t <dy_t, y_t> + <dh_final, h_final>
 * with respect to every input, for given dy (B,L,H,R,P) and dh_final (B,H,N,P)
 * (nullable: zero).  It is the exact derivative of the forward recurrence,
 * taken step by step in reverse order of the same operations (the chain rule
 * written out; no other formula is involved):
 *
 *   h_final = R(phi_L) ht_L:     g_L = R(-phi_L) dh_final, and phi_L gets
 *                                <dh_final, J h_final> per pair (J = d/da R(a) R(-a));
 *   y_t[r] = Ct_t[r]^T ht_t:     dCt_t[r] = ht_t dy_t[r],  g_t += Ct_t[r] dy_t[r]^T;
 *   ht_t = alpha ht_{t-1} + beta Q_{t-1} + gamma Q_t  (Q_t = sum_r Bt_t[r] x_t[r]^T):
 *                                dalpha = <g_t, ht_{t-1}>, dbeta = <g_t, Q_{t-1}>,
 *                                dgamma = <g_t, Q_t>, dQ_t += gamma g_t,
 *                                dQ_{t-1} += beta g_t, g_{t-1} = alpha g_t;
 *   Q_t:                         dBt_t[r] = dQ_t x_t[r], dx_t[r] = dQ_t^T Bt_t[r];
 *   Bt = R(-phi) B, Ct likewise: dB = R(phi) dBt, and phi_t gets
 *                                dBt[2k] Bt[2k+1] - dBt[2k+1] Bt[2k] (+ the same for C);
 *   phi_t = phi_{t-1} + dt_t theta_t: the angle adjoint accumulates backwards,
 *                                dtheta_t = dt_t dphi_t, ddt_t += <theta_t, dphi_t>;
 *   alpha = exp(dt A), beta = (1 - lam) dt alpha, gamma = lam dt: the scalar
 *                                chain rule.
 * The token before the first (prev_B, prev_x) sits at angle 0, so its
 * gradients need no rotation; dh0 is g_0.
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t B, L, H, P, N, R;
  const double *x, *Bm, *Cm, *dt, *A, *lam, *theta, *h0, *prev_B, *prev_x, *dy, *dhf;
  double *dx, *dB, *dC, *ddt, *dA, *dlam, *dtheta, *dh0, *dprev_B, *dprev_x;
  int64_t slice_begin, slice_end;
} bwd_job;

static void bwd_slice(const bwd_job* j, int64_t bh) {
  const int64_t L = j->L, H = j->H, P = j->P, N = j->N, R = j->R, K = N / 2, NP = N * P;
  const int64_t b = bh / H, h = bh % H;
  /* forward pass, keeping what the reverse pass needs */
  double* hs = (double*)calloc((size_t)((L + 1) * NP), sizeof(double)); /* ht_0 .. ht_L */
  double* phi = (double*)calloc((size_t)((L + 1) * K), sizeof(double));  /* phi_0 .. phi_L */
  double* Bt = (double*)calloc((size_t)((L + 1) * R * N), sizeof(double)); /* row 0: prev_B */
  double* Ct = (double*)calloc((size_t)((L + 1) * R * N), sizeof(double));
  double* xs = (double*)calloc((size_t)((L + 1) * R * P), sizeof(double)); /* row 0: prev_x */
  if (j->h0) memcpy(hs, j->h0 + bh * NP, sizeof(double) * (size_t)NP);
  if (j->prev_B && j->prev_x) {
    memcpy(Bt, j->prev_B + bh * R * N, sizeof(double) * (size_t)(R * N));
    memcpy(xs, j->prev_x + bh * R * P, sizeof(double) * (size_t)(R * P));
  }
  for (int64_t t = 1; t <= L; ++t) {
    const int64_t tok = (b * L + (t - 1)) * H + h;
    const double dt = j->dt[tok], alpha = exp(dt * j->A[tok]);
    const double beta = (1.0 - j->lam[tok]) * dt * alpha, gamma = j->lam[tok] * dt;
    for (int64_t k = 0; k < K; ++k) phi[t * K + k] = phi[(t - 1) * K + k] + dt * j->theta[tok * K + k];
    memcpy(xs + t * R * P, j->x + tok * R * P, sizeof(double) * (size_t)(R * P));
    for (int64_t r = 0; r < R; ++r)
      for (int64_t k = 0; k < K; ++k) {
        const int64_t i = r * N + 2 * k;
        rot(-phi[t * K + k], j->Bm[tok * R * N + i], j->Bm[tok * R * N + i + 1], &Bt[t * R * N + i], &Bt[t * R * N + i + 1]);
        rot(-phi[t * K + k], j->Cm[tok * R * N + i], j->Cm[tok * R * N + i + 1], &Ct[t * R * N + i], &Ct[t * R * N + i + 1]);
      }
    for (int64_t n = 0; n < N; ++n)
      for (int64_t p = 0; p < P; ++p) {
        double qp = 0.0, qc = 0.0;
        for (int64_t r = 0; r < R; ++r) {
          qp += Bt[(t - 1) * R * N + r * N + n] * xs[(t - 1) * R * P + r * P + p];
          qc += Bt[t * R * N + r * N + n] * xs[t * R * P + r * P + p];
        }
        hs[t * NP + n * P + p] = alpha * hs[(t - 1) * NP + n * P + p] + beta * qp + gamma * qc;
      }
  }

  /* reverse pass */
  double* g = (double*)calloc((size_t)NP, sizeof(double));      /* adjoint of ht_t */
  double* dQn = (double*)calloc((size_t)NP, sizeof(double));    /* beta_{t+1} g_{t+1}: pending part of dQ_t */
  double* dQ = (double*)calloc((size_t)NP, sizeof(double));
  double* dphi = (double*)calloc((size_t)K, sizeof(double));    /* running angle adjoint */
  double* dBt = (double*)calloc((size_t)(R * N), sizeof(double));
  double* dCt = (double*)calloc((size_t)(R * N), sizeof(double));
  if (j->dhf) {
    const double* dh = j->dhf + bh * NP;
    for (int64_t k = 0; k < K; ++k) {
      const double a = phi[L * K + k], c = cos(a), s = sin(a);
      for (int64_t p = 0; p < P; ++p) {
        const double du = dh[(2 * k) * P + p], dv = dh[(2 * k + 1) * P + p];
        const double u = hs[L * NP + (2 * k) * P + p], v = hs[L * NP + (2 * k + 1) * P + p];
        /* h_final = R(a) (u, v): adjoint R(-a) (du, dv); d/da R(a)(u,v) = (-s u - c v, c u - s v) */
        g[(2 * k) * P + p] = c * du + s * dv;
        g[(2 * k + 1) * P + p] = -s * du + c * dv;
        dphi[k] += du * (-s * u - c * v) + dv * (c * u - s * v);
      }
    }
  }
  for (int64_t t = L; t >= 1; --t) {
    const int64_t tok = (b * L + (t - 1)) * H + h;
    const double dt = j->dt[tok], A = j->A[tok], lam = j->lam[tok], alpha = exp(dt * A);
    const double beta = (1.0 - lam) * dt * alpha, gamma = lam * dt;
    const double* dyt = j->dy + tok * R * P;
    /* y_t */
    for (int64_t r = 0; r < R; ++r)
      for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t p = 0; p < P; ++p) acc += hs[t * NP + n * P + p] * dyt[r * P + p];
        dCt[r * N + n] = acc;
      }
    for (int64_t n = 0; n < N; ++n)
      for (int64_t p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int64_t r = 0; r < R; ++r) acc += Ct[t * R * N + r * N + n] * dyt[r * P + p];
        g[n * P + p] += acc;
      }
    /* ht_t = alpha ht_{t-1} + beta Q_{t-1} + gamma Q_t */
    double dalpha = 0.0, dbeta = 0.0, dgamma = 0.0;
    for (int64_t n = 0; n < N; ++n)
      for (int64_t p = 0; p < P; ++p) {
        double qp = 0.0, qc = 0.0;
        for (int64_t r = 0; r < R; ++r) {
          qp += Bt[(t - 1) * R * N + r * N + n] * xs[(t - 1) * R * P + r * P + p];
          qc += Bt[t * R * N + r * N + n] * xs[t * R * P + r * P + p];
        }
        const double gg = g[n * P + p];
        dalpha += gg * hs[(t - 1) * NP + n * P + p];
        dbeta += gg * qp;
        dgamma += gg * qc;
        dQ[n * P + p] = gamma * gg + dQn[n * P + p]; /* complete dQ_t */
#if ORACLE_MUTANT == 10
        dQn[n * P + p] = 0.0; /* mutant: the trapezoid term's adjoint is dropped */
#else
        dQn[n * P + p] = beta * gg;                  /* pending part of dQ_{t-1} */
#endif
        g[n * P + p] = alpha * gg;                   /* becomes g_{t-1} */
      }
    /* Q_t = sum_r Bt_t[r] x_t[r]^T */
    double* dxt = j->dx + tok * R * P;
    for (int64_t r = 0; r < R; ++r) {
      for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t p = 0; p < P; ++p) acc += dQ[n * P + p] * xs[t * R * P + r * P + p];
        dBt[r * N + n] = acc;
      }
      for (int64_t p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += dQ[n * P + p] * Bt[t * R * N + r * N + n];
        dxt[r * P + p] = acc;
      }
    }
    /* rotations of B and C, and the angle adjoint */
    double* dBo = j->dB + tok * R * N;
    double* dCo = j->dC + tok * R * N;
    for (int64_t k = 0; k < K; ++k) {
      const double a = phi[t * K + k];
      double dp = 0.0;
      for (int64_t r = 0; r < R; ++r) {
        const int64_t i = r * N + 2 * k;
        rot(a, dBt[i], dBt[i + 1], &dBo[i], &dBo[i + 1]);
        rot(a, dCt[i], dCt[i + 1], &dCo[i], &dCo[i + 1]);
#if ORACLE_MUTANT == 11
        dp -= dBt[i] * Bt[t * R * N + i + 1] - dBt[i + 1] * Bt[t * R * N + i]; /* mutant: sign of B's angle term */
#else
        dp += dBt[i] * Bt[t * R * N + i + 1] - dBt[i + 1] * Bt[t * R * N + i];
#endif
        dp += dCt[i] * Ct[t * R * N + i + 1] - dCt[i + 1] * Ct[t * R * N + i];
      }
      dphi[k] += dp;
    }
    /* scalars */
    double ddt = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      j->dtheta[tok * K + k] = dt * dphi[k];
      ddt += j->theta[tok * K + k] * dphi[k];
    }
    ddt += A * alpha * dalpha + ((1.0 - lam) * alpha + (1.0 - lam) * dt * A * alpha) * dbeta + lam * dgamma;
    j->ddt[tok] = ddt;
    j->dA[tok] = dt * alpha * dalpha + (1.0 - lam) * dt * dt * alpha * dbeta;
    j->dlam[tok] = -dt * alpha * dbeta + dt * dgamma;
  }
  if (j->dh0) memcpy(j->dh0 + bh * NP, g, sizeof(double) * (size_t)NP);
  if (j->dprev_B && j->prev_B) {
    /* dQ_0 = beta_1 g_1 (the pending part); prev sits at angle 0 */
    for (int64_t r = 0; r < R; ++r) {
      for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t p = 0; p < P; ++p) acc += dQn[n * P + p] * xs[r * P + p];
        j->dprev_B[(bh * R + r) * N + n] = acc;
      }
      for (int64_t p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += dQn[n * P + p] * Bt[r * N + n];
        j->dprev_x[(bh * R + r) * P + p] = acc;
      }
    }
  }
  free(hs); free(phi); free(Bt); free(Ct); free(xs);
  free(g); free(dQn); free(dQ); free(dphi); free(dBt); free(dCt);
}

static void* bwd_worker(void* arg) {
  bwd_job* j = (bwd_job*)arg;
  for (int64_t bh = j->slice_begin; bh < j->slice_end; ++bh) bwd_slice(j, bh);
  return NULL;
}

/* Returns 0 on success, -1 on bad arguments.  dh_final, h0, prev_B/prev_x
 * nullable; dh0 is written when non-NULL, dprev_B/dprev_x when prev_B is
 * given and they are non-NULL. */
int mamba3_oracle_backward(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t R,
                           const double* x, const double* Bm, const double* Cm,
                           const double* dt, const double* A, const double* lam, const double* theta,
                           const double* h0, const double* prev_B, const double* prev_x,
                           const double* dy, const double* dh_final,
                           double* dx, double* dB, double* dC, double* ddt, double* dA, double* dlam,
                           double* dtheta, double* dh0, double* dprev_B, double* dprev_x, int nthreads) {
  if (B <= 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || R <= 0 || (N % 2) != 0) return -1;
  if (L > 0 && (!x || !Bm || !Cm || !dt || !A || !lam || !theta || !dy || !dx || !dB || !dC || !ddt ||
                !dA || !dlam || !dtheta))
    return -1;
  const int64_t slices = B * H;
  const int nt = pick_threads(nthreads, slices);
  bwd_job* jobs = (bwd_job*)calloc((size_t)nt, sizeof(bwd_job));
  pthread_t* tids = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
  for (int i = 0; i < nt; ++i) {
    bwd_job* j = &jobs[i];
    j->B = B; j->L = L; j->H = H; j->P = P; j->N = N; j->R = R;
    j->x = x; j->Bm = Bm; j->Cm = Cm; j->dt = dt; j->A = A; j->lam = lam; j->theta = theta;
    j->h0 = h0; j->prev_B = prev_B; j->prev_x = prev_x; j->dy = dy; j->dhf = dh_final;
    j->dx = dx; j->dB = dB; j->dC = dC; j->ddt = ddt; j->dA = dA; j->dlam = dlam; j->dtheta = dtheta;
    j->dh0 = dh0; j->dprev_B = dprev_B; j->dprev_x = dprev_x;
    j->slice_begin = slices * i / nt;
    j->slice_end = slices * (i + 1) / nt;
  }
  for (int i = 1; i < nt; ++i) pthread_create(&tids[i], NULL, bwd_worker, &jobs[i]);
  bwd_worker(&jobs[0]);
  for (int i = 1; i < nt; ++i) pthread_join(tids[i], NULL);
  free(jobs); free(tids);
  return 0;
}

/* Cumulative-angle rotation on its own (linkstar.cloud/article/869, section
 * "第二刀", the RoPE form): phi_t = angle0 + sum_{s<=t} dt_s theta_s, then
 * B_rot = R(-phi_t) B_t and C_rot = R(-phi_t) C_t; angle_final = phi_L. */
int mamba3_oracle_rope_bc(int64_t B, int64_t L, int64_t H, int64_t N, int64_t R,
                          const double* Bm, const double* Cm, const double* dt, const double* theta,
                          const double* angle0, double* B_rot, double* C_rot, double* angle_final) {
  if (B <= 0 || L < 0 || H <= 0 || N <= 0 || R <= 0 || (N % 2) != 0) return -1;
  const int64_t K = N / 2;
  double* phi = (double*)malloc(sizeof(double) * (size_t)K);
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h) {
      for (int64_t k = 0; k < K; ++k) phi[k] = angle0 ? angle0[(b * H + h) * K + k] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        const int64_t tok = (b * L + t) * H + h;
        for (int64_t k = 0; k < K; ++k) phi[k] += dt[tok] * theta[tok * K + k];
        for (int64_t r = 0; r < R; ++r)
          for (int64_t k = 0; k < K; ++k) {
            const int64_t i0 = (tok * R + r) * N + 2 * k;
            rot(-phi[k], Bm[i0], Bm[i0 + 1], &B_rot[i0], &B_rot[i0 + 1]);
            rot(-phi[k], Cm[i0], Cm[i0 + 1], &C_rot[i0], &C_rot[i0 + 1]);
          }
      }
      if (angle_final)
        for (int64_t k = 0; k < K; ++k) angle_final[(b * H + h) * K + k] = phi[k];
    }
  free(phi);
  return 0;
}

int mamba3_oracle_version(void) { return 1000 + ORACLE_MUTANT; }
