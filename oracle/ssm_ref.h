/*
 * ssm_ref.h -- fp64 CPU oracle for the selective state-space scan.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously-correct
 * reference that the GPU path is checked against.  Only the test-suite, the
 * smoke check and the CPU-baseline leg of the benchmark load it; the product
 * path never calls it and shares no code, header or constant with it.
 *
 * Every buffer is a HOST pointer to contiguous row-major fp64 data owned by
 * the caller.  Layouts (dimension names follow the pages):
 *   u, delta, z, y        [batch, L, dim]
 *   B, C                  [batch, L, dstate]   (shared by every channel)
 *   A                     [dim, dstate]        (diagonal state matrix per channel)
 *   D, delta_bias         [dim]
 *   state / final_state   [batch, dim, dstate]
 * Nullable arguments: D (treated as 0), z (no gate), delta_bias (treated as 0),
 * final_state (not written).
 *
 * Return value: 0 on success, -1 on a bad argument (null required pointer or
 * a size <= 0).  Nothing is allocated that outlives a call.
 */
#ifndef SSM_REF_H
#define SSM_REF_H

#ifdef __cplusplus
extern "C" {
#endif

/* Selective scan over a whole sequence from a zero state.
 *   "The State That Must Remember Everything", Part 2, "The Equation":
 *       h_t = Abar h_{t-1} + Bbar u_t,   y_t = C h_t
 *   with Abar = exp(delta_t * A) (exponential-Euler, Part 7) and
 *   Bbar u_t = delta_t * B_t * u_t; delta, B and C are per token
 *   ("State Space Models and the Post-Transformer Era", "The Selection
 *   Mechanism").  The D*u skip comes from the continuous model
 *   y = Cx + Du (same page, "From Convolutions to State Spaces: S4").
 *   delta_t = softplus(delta_raw + bias) when softplus_flag != 0, and the
 *   output is multiplied by SiLU(z) when z is given.
 * nthreads >= 1 splits the independent (batch, channel) recurrences over
 * POSIX threads; the arithmetic of each recurrence is unchanged, so the
 * result does not depend on nthreads. */
int ssm_ref_scan_fwd(const double* u, const double* delta, const double* A,
                     const double* B, const double* C, const double* D,
                     const double* z, const double* delta_bias, int softplus_flag,
                     double* y, double* final_state,
                     long batch, long L, long dim, long dstate, int nthreads);

/* The same scan from given initial states and/or over packed sequences.
 *   initial_state (NULL: zero): h_{-1} for each recurrence, [rows][dim][dstate],
 *   so the scan continues a state handed on by an earlier call ("Mamba is
 *   attention all you really need, part 2", "The relay": a chunk starts from
 *   whatever state it is handed).
 *   cu_seqlens (NULL: none): batch must be 1; sequence s is tokens
 *   cu_seqlens[s] .. cu_seqlens[s+1]-1, each its own recurrence from its own
 *   initial state; rows = nseq, and final_state is [nseq][dim][dstate].
 *   cu_seqlens[0] = 0, nondecreasing, cu_seqlens[nseq] = L (else -1). */
int ssm_ref_scan_fwd_ex(const double* u, const double* delta, const double* A,
                        const double* B, const double* C, const double* D,
                        const double* z, const double* delta_bias, int softplus_flag,
                        const double* initial_state, const long* cu_seqlens, long nseq,
                        double* y, double* final_state,
                        long batch, long L, long dim, long dstate, int nthreads);

/* The same scan (and the same arguments) with the trapezoidal three-term
 * recurrence of Mamba-3 ("The State That Must Remember Everything", Part 7,
 * "Mamba-3 (2026)", item 1):
 *       h_t = alpha_t h_{t-1} + beta_t B_{t-1} u_{t-1} + gamma_t B_t u_t
 *   The page calls it a trapezoidal variant of the exponential-Euler rule and
 *   leaves alpha, beta, gamma undefined.  Reading: the trapezoidal rule
 *   applied to the step's input integral, whose integrand at the step's start
 *   has faded by exp(delta_t A) and at its end not at all:
 *       alpha_t = exp(delta_t A),  beta_t = delta_t/2 * exp(delta_t A),
 *       gamma_t = delta_t/2.
 *   At the first token of a recurrence (a batch row, or a packed sequence)
 *   the previous input is zero, also when an initial state is given.  The
 *   readout, skip and gate are those of ssm_ref_scan_fwd.
 *   Parity partly pinned: the tests fix this reading (impulse response,
 *   closed form, second-order convergence), not that it is the paper's. */
int ssm_ref_scan_trap_fwd_ex(const double* u, const double* delta, const double* A,
                             const double* B, const double* C, const double* D,
                             const double* z, const double* delta_bias, int softplus_flag,
                             const double* initial_state, const long* cu_seqlens, long nseq,
                             double* y, double* final_state,
                             long batch, long L, long dim, long dstate, int nthreads);

/* Backward of ssm_ref_scan_fwd_ex without packed sequences: the gradients of
 *   sum(y * dy) + sum(final_state * dfinal_state)
 * with respect to every input, by the adjoint recurrence run backwards over
 * each (row, channel) after a forward pass that keeps its states.
 *   dy, du, ddelta, dz: [batch, L, dim];  dB, dC: [batch, L, dstate];
 *   dA: [dim, dstate];  dD, ddelta_bias: [dim];
 *   dfinal_state, initial_state, dinitial_state: [batch, dim, dstate].
 * dfinal_state, initial_state (NULL: zero) and dinitial_state are optional;
 * dD, dz and ddelta_bias are required exactly when D, z and delta_bias are
 * given.  Sums over rows or channels (dA, dB, dC, dD, ddelta_bias) are added
 * per worker and then across workers in worker order, so a result depends
 * on nthreads only through that order.  Returns 0, -1 on bad arguments, -2
 * when its work buffers cannot be allocated. */
int ssm_ref_scan_bwd(const double* u, const double* delta, const double* A,
                     const double* B, const double* C, const double* D,
                     const double* z, const double* delta_bias, int softplus_flag,
                     const double* initial_state, const double* dy, const double* dfinal_state,
                     double* du, double* ddelta, double* dA, double* dB, double* dC,
                     double* dD, double* dz, double* ddelta_bias, double* dinitial_state,
                     long batch, long L, long dim, long dstate, int nthreads);

/* The same backward for the trapezoidal three-term recurrence of
 * ssm_ref_scan_trap_fwd_ex (batch rows, no packed sequences); arguments as
 * ssm_ref_scan_bwd. */
int ssm_ref_scan_trap_bwd(const double* u, const double* delta, const double* A,
                          const double* B, const double* C, const double* D,
                          const double* z, const double* delta_bias, int softplus_flag,
                          const double* initial_state, const double* dy, const double* dfinal_state,
                          double* du, double* ddelta, double* dA, double* dB, double* dC,
                          double* dD, double* dz, double* ddelta_bias, double* dinitial_state,
                          long batch, long L, long dim, long dstate, int nthreads);

/* One recurrent (decode) step from the given state, updated in place.
 *   u, delta, z, y: [batch, dim];  B, C: [batch, dstate];
 *   state: [batch, dim, dstate].  Same arithmetic as one step of the scan. */
int ssm_ref_state_update(double* state, const double* u, const double* delta,
                         const double* A, const double* B, const double* C,
                         const double* D, const double* z, const double* delta_bias,
                         int softplus_flag, double* y,
                         long batch, long dim, long dstate);

/* The fade-and-add composition "(a1,b1) then (a2,b2) = (a1 a2, a2 b1 + b2)"
 * ("Mamba is attention all you really need, part 2", "The relay"),
 * applied elementwise to n pairs. */
void ssm_ref_pair_then(long n, const double* a1, const double* b1,
                       const double* a2, const double* b2,
                       double* a_out, double* b_out);

/* Scalar helpers used by the scan, exported so tests can pin them. */
double ssm_ref_softplus(double x);  /* log(1 + e^x) */
double ssm_ref_silu(double z);      /* z * sigmoid(z) */

#ifdef __cplusplus
}
#endif
#endif
