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
