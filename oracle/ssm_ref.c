/*
 * ssm_ref.c -- fp64 CPU oracle for the selective state-space scan.
 *
 * TEST INFRASTRUCTURE ONLY: the reference the GPU path is checked against.
 * Plain sequential C99, double precision, no SIMD intrinsics, no fast-math.
 * It shares no code with the GPU path.
 *
 * What it computes (notation of the pages):
 *   - the discrete recurrence and readout h_t = Abar h_{t-1} + Bbar u_t,
 *     y_t = C h_t  ("The State That Must Remember Everything", Part 2,
 *     "The Equation"), with no nonlinearity between steps;
 *   - Abar = exp(delta * A) for the diagonal A of each channel and
 *     Bbar = delta * B, the exponential-Euler reading of the discretisation
 *     that the same page (Part 7) attributes to Mamba-1/2;
 *   - delta, B and C given per token ("State Space Models and the
 *     Post-Transformer Era", "The Selection Mechanism");
 *   - the skip term D*u of the continuous model y = Cx + Du (same page,
 *     "From Convolutions to State Spaces: S4");
 *   - y_t reads the state AFTER token t has been written into it;
 *   - optional softplus on delta (with a per-channel bias) and an optional
 *     SiLU(z) gate on the output;
 *   - and, for Mamba-3, the three-term trapezoidal recurrence (same page,
 *     Part 7, "Mamba-3 (2026)"; alpha, beta, gamma as read in ssm_ref.h).
 */
#include "ssm_ref.h"

#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdlib.h>

double ssm_ref_softplus(double x) {
  /* log(1 + e^x), written so that e^x never overflows:
   * for x > 0, log(1 + e^x) = x + log(1 + e^-x). */
  if (x > 0.0) return x + log1p(exp(-x));
  return log1p(exp(x));
}

double ssm_ref_silu(double z) {
  /* z * sigmoid(z) = z / (1 + e^-z) */
  return z / (1.0 + exp(-z));
}

void ssm_ref_pair_then(long n, const double* a1, const double* b1,
                       const double* a2, const double* b2,
                       double* a_out, double* b_out) {
  for (long i = 0; i < n; ++i) {
    double a = a1[i] * a2[i];
    double b = a2[i] * b1[i] + b2[i];
    a_out[i] = a;
    b_out[i] = b;
  }
}

/* delta for one (token, channel): raw value plus bias, then softplus. */
static double step_delta(double raw, const double* bias, long d, int softplus_flag) {
  double x = raw + (bias ? bias[d] : 0.0);
  return softplus_flag ? ssm_ref_softplus(x) : x;
}

/* One recurrence step for one channel d: updates h[0:N] in place and
 * returns the gated output.  Bt, Ct point at this token's B and C rows. */
static double one_step(double* h, double ut, double dt_raw, const double* zt,
                       const double* Arow, const double* Bt, const double* Ct,
                       const double* D, const double* bias, long d, long N,
                       int softplus_flag) {
  double delta = step_delta(dt_raw, bias, d, softplus_flag);
  double acc = 0.0;
  for (long n = 0; n < N; ++n) {
    double abar = exp(delta * Arow[n]);        /* fade */
    double bbar_u = delta * Bt[n] * ut;        /* add */
    h[n] = abar * h[n] + bbar_u;               /* h_t = Abar h_{t-1} + Bbar u_t */
    acc += Ct[n] * h[n];                       /* y_t = C_t . h_t */
  }
  double v = acc + (D ? D[d] : 0.0) * ut;      /* + D u_t */
  if (zt) v = v * ssm_ref_silu(*zt);           /* gate */
  return v;
}

/* One step of the trapezoidal three-term recurrence for channel d:
 *   h_t = alpha_t h_{t-1} + beta_t B_{t-1} u_{t-1} + gamma_t B_t u_t
 * with alpha_t = exp(delta_t A), beta_t = delta_t/2 exp(delta_t A),
 * gamma_t = delta_t/2.  Bprev is the previous token's B row (NULL at the
 * first token of a recurrence, whose previous input is zero) and uprev its
 * input. */
static double trap_step(double* h, double ut, double dt_raw, const double* zt,
                        const double* Arow, const double* Bprev, double uprev,
                        const double* Bt, const double* Ct, const double* D,
                        const double* bias, long d, long N, int softplus_flag) {
  double delta = step_delta(dt_raw, bias, d, softplus_flag);
  double acc = 0.0;
  for (long n = 0; n < N; ++n) {
    double alpha = exp(delta * Arow[n]);
    double beta = 0.5 * delta * alpha;
    double gamma = 0.5 * delta;
    double prev_in = Bprev ? beta * Bprev[n] * uprev : 0.0;
    h[n] = alpha * h[n] + prev_in + gamma * Bt[n] * ut;
    acc += Ct[n] * h[n];                       /* y_t = C_t . h_t */
  }
  double v = acc + (D ? D[d] : 0.0) * ut;
  if (zt) v = v * ssm_ref_silu(*zt);
  return v;
}

typedef struct {
  const double *u, *delta, *A, *B, *C, *D, *z, *bias;
  int softplus_flag;
  double *y, *final_state;
  long batch, L, dim, N;
  const double* h0;      /* initial states [rows][dim][N], or NULL for zero */
  const long* cu;        /* packed sequences: row r is tokens cu[r] .. cu[r+1]-1 of batch row 0 */
  long rows;             /* batch rows, or sequences when cu is given */
  int trapezoid;         /* the three-term recurrence instead of exponential-Euler */
  long first, last; /* range of flattened (row, d) channels for this worker */
} scan_job;

static void scan_channels(const scan_job* j) {
  double hbuf[4096];
  for (long rd = j->first; rd < j->last; ++rd) {
    long r = rd / j->dim, d = rd % j->dim;
    /* the tokens of this recurrence: a whole batch row, or one packed sequence of row 0 */
    long b = j->cu ? 0 : r;
    long t0 = j->cu ? j->cu[r] : 0, t1 = j->cu ? j->cu[r + 1] : j->L;
    double* h = hbuf;
    for (long n = 0; n < j->N; ++n)                /* the given state, else zero */
      h[n] = j->h0 ? j->h0[(r * j->dim + d) * j->N + n] : 0.0;
    const double* Bprev = NULL;                   /* trapezoidal rule: the previous token's B and u */
    double uprev = 0.0;
    for (long t = t0; t < t1; ++t) {
      long io = (b * j->L + t) * j->dim + d;      /* [batch, L, dim] */
      long bc = (b * j->L + t) * j->N;            /* [batch, L, dstate] */
      if (j->trapezoid) {
        j->y[io] = trap_step(h, j->u[io], j->delta[io], j->z ? &j->z[io] : NULL,
                             &j->A[d * j->N], Bprev, uprev, &j->B[bc], &j->C[bc], j->D,
                             j->bias, d, j->N, j->softplus_flag);
        Bprev = &j->B[bc];
        uprev = j->u[io];
      } else {
        j->y[io] = one_step(h, j->u[io], j->delta[io], j->z ? &j->z[io] : NULL,
                            &j->A[d * j->N], &j->B[bc], &j->C[bc], j->D, j->bias, d,
                            j->N, j->softplus_flag);
      }
    }
    if (j->final_state)
      for (long n = 0; n < j->N; ++n) j->final_state[(r * j->dim + d) * j->N + n] = h[n];
  }
}

static void* scan_worker(void* arg) {
  scan_channels((const scan_job*)arg);
  return NULL;
}

int ssm_ref_scan_fwd(const double* u, const double* delta, const double* A,
                     const double* B, const double* C, const double* D,
                     const double* z, const double* delta_bias, int softplus_flag,
                     double* y, double* final_state,
                     long batch, long L, long dim, long dstate, int nthreads) {
  return ssm_ref_scan_fwd_ex(u, delta, A, B, C, D, z, delta_bias, softplus_flag, NULL, NULL, 0,
                             y, final_state, batch, L, dim, dstate, nthreads);
}

static int scan_rows(const double* u, const double* delta, const double* A,
                     const double* B, const double* C, const double* D,
                     const double* z, const double* delta_bias, int softplus_flag,
                     const double* initial_state, const long* cu_seqlens, long nseq,
                     double* y, double* final_state,
                     long batch, long L, long dim, long dstate, int nthreads, int trapezoid) {
  if (!u || !delta || !A || !B || !C || !y) return -1;
  if (batch <= 0 || L <= 0 || dim <= 0 || dstate <= 0 || dstate > 4096) return -1;
  long rows = batch;
  if (cu_seqlens) {
    if (batch != 1 || nseq <= 0 || cu_seqlens[0] != 0 || cu_seqlens[nseq] != L) return -1;
    for (long s = 0; s < nseq; ++s)
      if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
    rows = nseq;
  }
  long channels = rows * dim;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > channels) nthreads = (int)channels;

  scan_job jobs[256];
  pthread_t tids[256];
  int running[256];
  for (int i = 0; i < nthreads; ++i) {
    scan_job j = {u, delta, A, B, C, D, z, delta_bias, softplus_flag, y, final_state,
                  batch, L, dim, dstate, initial_state, cu_seqlens, rows, trapezoid,
                  channels * i / nthreads, channels * (i + 1) / nthreads};
    jobs[i] = j;
  }
  if (nthreads == 1) {
    scan_channels(&jobs[0]);
    return 0;
  }
  for (int i = 0; i < nthreads; ++i) {
    running[i] = pthread_create(&tids[i], NULL, scan_worker, &jobs[i]) == 0;
    if (!running[i]) scan_channels(&jobs[i]); /* no thread: do this share here */
  }
  for (int i = 0; i < nthreads; ++i)
    if (running[i]) pthread_join(tids[i], NULL);
  return 0;
}

int ssm_ref_scan_fwd_ex(const double* u, const double* delta, const double* A,
                        const double* B, const double* C, const double* D,
                        const double* z, const double* delta_bias, int softplus_flag,
                        const double* initial_state, const long* cu_seqlens, long nseq,
                        double* y, double* final_state,
                        long batch, long L, long dim, long dstate, int nthreads) {
  return scan_rows(u, delta, A, B, C, D, z, delta_bias, softplus_flag, initial_state, cu_seqlens, nseq,
                   y, final_state, batch, L, dim, dstate, nthreads, 0);
}

int ssm_ref_scan_trap_fwd_ex(const double* u, const double* delta, const double* A,
                             const double* B, const double* C, const double* D,
                             const double* z, const double* delta_bias, int softplus_flag,
                             const double* initial_state, const long* cu_seqlens, long nseq,
                             double* y, double* final_state,
                             long batch, long L, long dim, long dstate, int nthreads) {
  return scan_rows(u, delta, A, B, C, D, z, delta_bias, softplus_flag, initial_state, cu_seqlens, nseq,
                   y, final_state, batch, L, dim, dstate, nthreads, 1);
}

int ssm_ref_state_update(double* state, const double* u, const double* delta,
                         const double* A, const double* B, const double* C,
                         const double* D, const double* z, const double* delta_bias,
                         int softplus_flag, double* y,
                         long batch, long dim, long dstate) {
  if (!state || !u || !delta || !A || !B || !C || !y) return -1;
  if (batch <= 0 || dim <= 0 || dstate <= 0) return -1;
  for (long b = 0; b < batch; ++b) {
    for (long d = 0; d < dim; ++d) {
      long io = b * dim + d;                       /* [batch, dim] */
      y[io] = one_step(&state[io * dstate], u[io], delta[io], z ? &z[io] : NULL,
                       &A[d * dstate], &B[b * dstate], &C[b * dstate], D, delta_bias, d,
                       dstate, softplus_flag);
    }
  }
  return 0;
}

/*
 * Backward pass of the two-term scan (batch rows, optional initial state):
 * the gradients of  sum_t y_t dy_t + sum_n final_state[n] dfinal_state[n]
 * with respect to every input, by the adjoint of the recurrence, one
 * (row, channel) at a time.  The pages only say that training recomputes the
 * states instead of storing them ("Mamba is attention all you really need,
 * part 2", "Keeping the pad on the desk"); the gradients themselves follow
 * from the forward definition above.  With lambda_t the gradient reaching
 * h_t (from y_t, and from h_{t+1} through the fade a_{t+1}):
 *   lambda_{L-1} = dfinal_state + C_{L-1} dv_{L-1},
 *   lambda_t     = C_t dv_t + a_{t+1} lambda_{t+1},      dv_t = dy_t SiLU(z_t),
 * and for h_t = a_t h_{t-1} + Delta_t u_t B_t, a_t = exp(Delta_t A):
 *   dDelta_t = sum_n lambda_t[n] (A[n] a_t[n] h_{t-1}[n] + u_t B_t[n]),
 *   dA[n]   += lambda_t[n] Delta_t a_t[n] h_{t-1}[n],
 *   du_t     = sum_n lambda_t[n] Delta_t B_t[n] + D dv_t,
 *   dB_t[n] += lambda_t[n] Delta_t u_t,   dC_t[n] += dv_t h_t[n],
 *   dz_t     = dy_t v_t SiLU'(z_t),       dD += dv_t u_t,
 *   ddelta_t = dDelta_t sigmoid(x_t) (softplus' = sigmoid; 1 without softplus),
 *   dbias   += ddelta_t,                  dinitial_state = a_0 lambda_0.
 * With the trapezoidal rule (ssm_ref_scan_trap_bwd), h_t = a_t h_{t-1} +
 * beta_t B_{t-1} u_{t-1} + gamma_t B_t u_t with beta_t = Delta_t/2 a_t and
 * gamma_t = Delta_t/2 (no previous term at a row's first token), so besides
 * the fade's terms
 *   dDelta_t += sum_n lambda_t[n] (B_t u_t / 2 + B_{t-1} u_{t-1} (a_t/2 + Delta_t/2 A a_t)),
 *   dA[n]   += lambda_t[n] B_{t-1}[n] u_{t-1} Delta_t^2/2 a_t[n],
 * and the input terms reach both tokens: du_t and dB_t through gamma_t,
 * du_{t-1} and dB_{t-1} through beta_t.
 * dB, dC, dA, dD and dbias sum over channels or rows: each worker sums its
 * own share, and the shares are added in worker order (deterministic).
 */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

typedef struct {
  const double *u, *delta, *A, *B, *C, *D, *z, *bias, *h0, *dy, *dfs;
  int softplus_flag;
  int trapezoid;                         /* the three-term recurrence of ssm_ref_scan_trap_fwd_ex */
  long batch, L, dim, N;
  double *du, *ddelta, *dz, *dinit;     /* per (row, channel): written directly */
  double *dA, *dB, *dC, *dD, *dbias;    /* this worker's partial sums */
  double* work;                          /* L*N + 2*L doubles: states, steps, pre-gate outputs */
  long first, last;
  int ok;
} bwd_job;

static void bwd_channels(bwd_job* j) {
  const long L = j->L, N = j->N, dim = j->dim;
  double* hs = j->work;            /* h_t[n] at hs[t*N + n] */
  double* dls = hs + L * N;        /* Delta_t */
  double* vs = dls + L;            /* v_t, before the gate */
  double lam[4096], hprev[4096];
  for (long rd = j->first; rd < j->last; ++rd) {
    const long b = rd / dim, d = rd % dim;
    const double* Ad = &j->A[d * N];
    /* forward, keeping every state */
    for (long n = 0; n < N; ++n) hprev[n] = j->h0 ? j->h0[(b * dim + d) * N + n] : 0.0;
    for (long t = 0; t < L; ++t) {
      const long io = (b * L + t) * dim + d, bc = (b * L + t) * N;
      const double dl = step_delta(j->delta[io], j->bias, d, j->softplus_flag);
      const double* hp = t ? &hs[(t - 1) * N] : hprev;
      double v = 0.0;
      for (long n = 0; n < N; ++n) {
        const double a = exp(dl * Ad[n]);
        double h;
        if (j->trapezoid) {   /* the previous token's input (none at a row's first token), then this one's */
          const double prev_in = t ? 0.5 * dl * a * j->B[bc - N + n] * j->u[io - dim] : 0.0;
          h = a * hp[n] + prev_in + 0.5 * dl * j->B[bc + n] * j->u[io];
        } else {
          h = a * hp[n] + dl * j->u[io] * j->B[bc + n];
        }
        hs[t * N + n] = h;
        v += j->C[bc + n] * h;
      }
      dls[t] = dl;
      vs[t] = v + (j->D ? j->D[d] * j->u[io] : 0.0);
    }
    /* backward */
    for (long n = 0; n < N; ++n) lam[n] = j->dfs ? j->dfs[(b * dim + d) * N + n] : 0.0;
    double du_next = 0.0;   /* trapezoidal rule: the part of du_t that step t+1 contributes */
    for (long t = L - 1; t >= 0; --t) {
      const long io = (b * L + t) * dim + d, bc = (b * L + t) * N;
      const double dl = dls[t], ut = j->u[io];
      double dv = j->dy[io];
      if (j->z) {
        const double zt = j->z[io], s = sigmoid(zt);
        j->dz[io] = j->dy[io] * vs[t] * s * (1.0 + zt * (1.0 - s));
        dv = j->dy[io] * zt * s;
      }
      double du = j->D ? j->D[d] * dv : 0.0, ddl = 0.0;
      du += du_next;
      du_next = 0.0;
      if (j->D) j->dD[d] += dv * ut;
      const double* hp = t ? &hs[(t - 1) * N] : hprev;
      for (long n = 0; n < N; ++n) {
        lam[n] += j->C[bc + n] * dv;
        j->dC[bc + n] += dv * hs[t * N + n];
        const double a = exp(dl * Ad[n]);
        if (j->trapezoid) {
          /* h_t = a h_{t-1} + (dl/2) a B_{t-1} u_{t-1} + (dl/2) B_t u_t */
          ddl += lam[n] * (Ad[n] * a * hp[n] + 0.5 * ut * j->B[bc + n]);
          j->dA[d * N + n] += lam[n] * dl * a * hp[n];
          du += lam[n] * 0.5 * dl * j->B[bc + n];
          j->dB[bc + n] += lam[n] * 0.5 * dl * ut;
          if (t) {
            const double bu = j->B[bc - N + n] * j->u[io - dim];     /* B_{t-1} u_{t-1} */
            ddl += lam[n] * bu * (0.5 * a + 0.5 * dl * Ad[n] * a);   /* d beta / d delta */
            j->dA[d * N + n] += lam[n] * bu * 0.5 * dl * dl * a;     /* d beta / d A */
            du_next += lam[n] * 0.5 * dl * a * j->B[bc - N + n];
            j->dB[bc - N + n] += lam[n] * 0.5 * dl * a * j->u[io - dim];
          }
        } else {
          ddl += lam[n] * (Ad[n] * a * hp[n] + ut * j->B[bc + n]);
          j->dA[d * N + n] += lam[n] * dl * a * hp[n];
          du += lam[n] * dl * j->B[bc + n];
          j->dB[bc + n] += lam[n] * dl * ut;
        }
        lam[n] *= a;                                   /* on to h_{t-1} */
      }
      j->du[io] = du;
      const double x = j->delta[io] + (j->bias ? j->bias[d] : 0.0);
      const double dx = j->softplus_flag ? ddl * sigmoid(x) : ddl;
      j->ddelta[io] = dx;
      if (j->bias) j->dbias[d] += dx;
    }
    if (j->dinit)
      for (long n = 0; n < N; ++n) j->dinit[(b * dim + d) * N + n] = lam[n];
  }
}

static void* bwd_worker(void* arg) {
  bwd_channels((bwd_job*)arg);
  return NULL;
}

static int scan_bwd_rows(const double* u, const double* delta, const double* A,
                         const double* B, const double* C, const double* D,
                         const double* z, const double* delta_bias, int softplus_flag,
                         const double* initial_state, const double* dy, const double* dfinal_state,
                         double* du, double* ddelta, double* dA, double* dB, double* dC,
                         double* dD, double* dz, double* ddelta_bias, double* dinitial_state,
                         long batch, long L, long dim, long dstate, int nthreads, int trapezoid) {
  if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC) return -1;
  if ((D && !dD) || (z && !dz) || (delta_bias && !ddelta_bias)) return -1;
  if (batch <= 0 || L <= 0 || dim <= 0 || dstate <= 0 || dstate > 4096) return -1;
  const long channels = batch * dim;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > channels) nthreads = (int)channels;
  const long nA = dim * dstate, nBC = batch * L * dstate;
  bwd_job jobs[256];
  pthread_t tids[256];
  int running[256];
  int rc = 0;
  for (int i = 0; i < nthreads; ++i) {
    bwd_job j = {u, delta, A, B, C, D, z, delta_bias, initial_state, dy, dfinal_state, softplus_flag, trapezoid,
                 batch, L, dim, dstate, du, ddelta, dz, dinitial_state,
                 (double*)calloc((size_t)nA, sizeof(double)), (double*)calloc((size_t)nBC, sizeof(double)),
                 (double*)calloc((size_t)nBC, sizeof(double)), (double*)calloc((size_t)dim, sizeof(double)),
                 (double*)calloc((size_t)dim, sizeof(double)),
                 (double*)malloc((size_t)(L * dstate + 2 * L) * sizeof(double)),
                 channels * i / nthreads, channels * (i + 1) / nthreads, 1};
    if (!j.dA || !j.dB || !j.dC || !j.dD || !j.dbias || !j.work) rc = -2;
    jobs[i] = j;
  }
  if (rc == 0) {
    for (int i = 0; i < nthreads; ++i) {
      running[i] = nthreads > 1 && pthread_create(&tids[i], NULL, bwd_worker, &jobs[i]) == 0;
      if (!running[i]) bwd_channels(&jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i)
      if (running[i]) pthread_join(tids[i], NULL);
    /* the workers' partial sums, in worker order */
    for (long e = 0; e < nA; ++e) {
      double s = 0.0;
      for (int i = 0; i < nthreads; ++i) s += jobs[i].dA[e];
      dA[e] = s;
    }
    for (long e = 0; e < nBC; ++e) {
      double sb = 0.0, sc = 0.0;
      for (int i = 0; i < nthreads; ++i) {
        sb += jobs[i].dB[e];
        sc += jobs[i].dC[e];
      }
      dB[e] = sb;
      dC[e] = sc;
    }
    for (long e = 0; e < dim; ++e) {
      double sd = 0.0, sbias = 0.0;
      for (int i = 0; i < nthreads; ++i) {
        sd += jobs[i].dD[e];
        sbias += jobs[i].dbias[e];
      }
      if (dD) dD[e] = sd;
      if (ddelta_bias) ddelta_bias[e] = sbias;
    }
  }
  for (int i = 0; i < nthreads; ++i) {
    free(jobs[i].dA);
    free(jobs[i].dB);
    free(jobs[i].dC);
    free(jobs[i].dD);
    free(jobs[i].dbias);
    free(jobs[i].work);
  }
  return rc;
}

int ssm_ref_scan_bwd(const double* u, const double* delta, const double* A,
                     const double* B, const double* C, const double* D,
                     const double* z, const double* delta_bias, int softplus_flag,
                     const double* initial_state, const double* dy, const double* dfinal_state,
                     double* du, double* ddelta, double* dA, double* dB, double* dC,
                     double* dD, double* dz, double* ddelta_bias, double* dinitial_state,
                     long batch, long L, long dim, long dstate, int nthreads) {
  return scan_bwd_rows(u, delta, A, B, C, D, z, delta_bias, softplus_flag, initial_state, dy, dfinal_state,
                       du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, batch, L, dim, dstate,
                       nthreads, 0);
}

int ssm_ref_scan_trap_bwd(const double* u, const double* delta, const double* A,
                          const double* B, const double* C, const double* D,
                          const double* z, const double* delta_bias, int softplus_flag,
                          const double* initial_state, const double* dy, const double* dfinal_state,
                          double* du, double* ddelta, double* dA, double* dB, double* dC,
                          double* dD, double* dz, double* ddelta_bias, double* dinitial_state,
                          long batch, long L, long dim, long dstate, int nthreads) {
  return scan_bwd_rows(u, delta, A, B, C, D, z, delta_bias, softplus_flag, initial_state, dy, dfinal_state,
                       du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, batch, L, dim, dstate,
                       nthreads, 1);
}
