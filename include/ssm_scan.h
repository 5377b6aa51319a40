/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective state-space scan.
 *
 * The operation.  For every batch b and channel d the library runs the
 * discretised, input-dependent state-space recurrence
 *     h_t = exp(delta_t * A[d,:]) (.) h_{t-1} + delta_t * B_t * u_t
 *     y_t = (C_t . h_t + D[d] * u_t) * SiLU(z_t)
 * with delta_t = softplus(delta_raw_t + delta_bias[d]) (or delta_raw_t +
 * delta_bias[d] when softplus_flag is 0).  Sources, by page title:
 *   - "The State That Must Remember Everything", Part 2 "The Equation":
 *     the discrete recurrence h_t = Abar h_{t-1} + Bbar u_t, y_t = C h_t, and
 *     the continuous model with the D u term; Part 7: Mamba-1/2 use an
 *     exponential-Euler discretisation (Abar = exp(delta A), Bbar = delta B);
 *     Part 3 "The Hardware-Aware Way Out": scan, fusion, state kept on chip.
 *   - "State Space Models and the Post-Transformer Era", "The Selection
 *     Mechanism": delta, B and C are computed per token; A is diagonal per
 *     channel ("Mamba-2 and Structured State Space Duality" contrasts it with
 *     Mamba-2's scalar A).
 *   - "Mamba is attention all you really need, part 2", "The relay": each
 *     step is a fade-and-add pair (a, b) and pairs compose as
 *     (a1,b1) then (a2,b2) = (a1 a2, a2 b1 + b2), which is what lets the
 *     sequence be cut into chunks that are scanned in parallel.
 * The SiLU(z) output gate, the softplus on delta and its per-channel bias
 * are the conventional Mamba block epilogue/prologue; the pages leave them
 * unspecified and this library takes that standard form.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library allocates and frees nothing and keeps no state between calls
 *     (beyond each device's compute-unit count, looked up once), so
 *     concurrent calls on different streams with their own workspaces are
 *     safe.
 *   - Launch plans balance the work over the current device's compute units;
 *     workspace sizes therefore depend on the device current when they are
 *     queried (the same device must be current for the call).  SSM_NUM_CU
 *     in the environment overrides the count (for tests of the plans).
 *   - Layouts are contiguous row-major:
 *       u, delta, z, y        [batch, L, dim]     (decode: [batch, dim])
 *       B, C                  [batch, L, dstate]  (decode: [batch, dstate]),
 *                             shared by all dim channels of a token
 *       A                     [dim, dstate]  fp32
 *       D, delta_bias         [dim]          fp32
 *       state, final_state    [batch, dim, dstate]  fp32
 *   - u, delta, z, B, C and y have dtype `dt` (fp32 or bf16); A, D,
 *     delta_bias and the state are fp32.  All arithmetic is fp32; bf16
 *     outputs are rounded to nearest even.
 *   - Work is enqueued on `stream` and the call returns at once; outputs are
 *     valid after the stream is synchronised.
 *   - Arguments are validated before any HIP call: a null required pointer,
 *     a size <= 0, an unknown dtype, a pointer not aligned to its element
 *     size, or a missing, too small or misaligned workspace gives
 *     SSM_ERR_INVALID_ARG; a dstate above 64 (above 256 for the decode
 *     step), a batch above 65535 or a token
 *     row (dim * element size) above 16 MiB gives SSM_ERR_UNSUPPORTED.
 *     Nothing is launched in either case.  A failed launch gives
 *     SSM_ERR_HIP.
 *     Input values are not inspected (NaN in gives NaN out).
 *   - Where a plan chains pieces of one sequence through the workspace (a
 *     piece starts from the state, or adjoint, that the piece before it
 *     hands on), each wait is bounded (about a third of a second).  Past the
 *     bound the piece goes on from NaN, so the outputs that depend on the
 *     lost hand-off are NaN rather than silently wrong, and the call's
 *     workspace records the time-out: ssm_workspace_status then returns
 *     SSM_ERR_HANDOFF_TIMEOUT.  It does not happen on a GPU that runs the
 *     call's workgroups.  Every workspace starts with a 256-byte header
 *     (status word, tickets, ready flags) that each call resets.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSM_OK = 0,
  SSM_ERR_INVALID_ARG = 1,
  SSM_ERR_UNSUPPORTED = 2,
  SSM_ERR_HIP = 3,
  SSM_ERR_HANDOFF_TIMEOUT = 4,
  SSM_ERR_SCRATCH_TOO_SMALL = 5
} ssm_status_t;

typedef enum { SSM_DTYPE_F32 = 0, SSM_DTYPE_BF16 = 1 } ssm_dtype_t;

/* Bytes of device workspace that ssm_scan_fwd needs for this shape (always
 * > 0 for a valid shape).  The workspace holds B and C repacked as fp32
 * records per group of states (about batch * L * 2 * dstate * 4 bytes) and,
 * when tiles of 64 channels are cut into chunks of the sequence, the state
 * carried into every chunk ("Mamba is attention all you really need, part
 * 2", "The relay": a chunk can start from the state the chunk before it hands
 * on), plus either the chunks' composed fade-and-add pairs or a few words of
 * ready flags.  Returns 0 for arguments ssm_scan_fwd would reject. */
size_t ssm_scan_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt);

/* Selective scan over a whole sequence, starting from a zero state.
 *   Required: u, delta, A, B, C, y.  Optional (NULL allowed): D (no skip
 *   term), z (no gate), delta_bias (zero bias), final_state (not written).
 *   final_state receives h_L, the state after the last token (before the
 *   gate, which only touches y).  workspace must point at workspace_bytes >=
 *   ssm_scan_workspace_size() bytes of device memory, 256-byte aligned,
 *   which the call overwrites and which must not be shared with a
 *   concurrent call.
 *   y must not alias any input. */
ssm_status_t ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                          const float* D, const void* z, const float* delta_bias, int softplus_flag,
                          void* y, float* final_state,
                          int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ssm_scan_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation, kernels and plan as ssm_scan_fwd with the same
 * arguments, bitwise the same outputs, but no workspace argument.  The
 * workspace is a static 32 MiB device array of the library, one per GPU
 * (each GPU holds it until the process ends); its device address is looked
 * up once per device, on the first call with that device current.  The call
 * itself allocates nothing: no hipMalloc, no hipFree, no allocating library
 * routine.  Every call on one GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (other streams, other threads) race and must
 * be serialised by the caller; sequential calls need nothing (each call
 * resets what must start at zero).  The stream must belong to the current
 * device.  ssm_workspace_status does not apply (there is no workspace to
 * pass); a lost hand-off still shows as NaN outputs.
 * Errors: as ssm_scan_fwd for the arguments; SSM_ERR_SCRATCH_TOO_SMALL when
 * the shape needs more than 32 MiB of workspace (ssm_scan_workspace_size
 * above 32 MiB: about batch * L above 250,000 tokens at dstate 16), nothing
 * launched; SSM_ERR_HIP if the array's address cannot be looked up. */
ssm_status_t ssm_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                  const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                  void* y, float* final_state,
                                  int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt,
                                  hipStream_t stream);

/* Workspace for ssm_scan_fwd_structured: the header words, for bf16 storage B
 * and C repacked as fp32 records (batch * L * 128 bytes, rounded up), and
 * three arrays of n_tiles * K * 64 * ns floats for the chunks' fade-and-add
 * pairs and carried-in states (n_tiles = batch * ceil(dim / 64), ns = 4, 8
 * or 16 states per lane, K the chunks per tile: about 10 * CUs / n_tiles).
 * Returns 0 for arguments the call would reject. */
size_t ssm_scan_fwd_structured_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate,
                                              ssm_dtype_t dt);

/* ssm_scan_fwd_ex (without packed sequences) for the structured state matrix
 *     A[d, n] = (n + 1) * A0[d],
 * a specialisation that the caller asserts by passing A0 [dim] (fp32) in
 * place of A: the fade of state n is then q^(n+1) with q = exp(delta_t
 * A0[d]), so a token costs one exp per channel and the fades follow by
 * repeated multiplication ("Mamba is attention all you really need, part 2",
 * "Keeping the pad on the desk": sixteen numbers per channel, one fade per
 * step; "The relay" for the chunk pairs).  The caller decides whether A has
 * this form (for instance once per weight, on the host); the library does not
 * inspect A.  The result equals ssm_scan_fwd_ex with that A up to fp32
 * rounding (the powers round differently from separate exps).
 *   dstate <= 16 (else SSM_ERR_UNSUPPORTED).  initial_state (NULL: zero):
 *   [batch, dim, dstate] fp32.  Everything else (arguments, layouts,
 *   ownership, errors) as ssm_scan_fwd; the workspace comes from
 *   ssm_scan_fwd_structured_workspace_size.  The plan has no chained
 *   hand-offs, so ssm_workspace_status always reports SSM_OK for it. */
ssm_status_t ssm_scan_fwd_structured(const void* u, const void* delta, const float* A0, const void* B,
                                     const void* C, const float* D, const void* z, const float* delta_bias,
                                     int softplus_flag, const float* initial_state, void* y, float* final_state,
                                     int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace for ssm_scan_fwd_ex: for nseq <= 0 (no packed sequences) the same
 * as ssm_scan_workspace_size; for nseq > 0 packed sequences (batch must be 1)
 * the packed B/C records and the order in which the sequences are launched
 * (longest first, nseq ints).  Returns 0 for arguments the call would
 * reject. */
size_t ssm_scan_fwd_ex_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate, int64_t nseq,
                                      ssm_dtype_t dt);

/* ssm_scan_fwd from given initial states and/or over packed sequences of
 * variable length ("Mamba is attention all you really need, part 2", "The
 * relay": a stretch of the sequence can start from whatever state it is
 * handed, so a long prompt can be scanned in pieces and a state handed on;
 * packed variable-length sequences as in "State Space Models and the
 * Post-Transformer Era", "Mamba-2 and Structured State Space Duality").
 *   initial_state (NULL: zero) is h_{-1} of every recurrence, fp32
 *   [rows, dim, dstate], rows = batch, or nseq with packed sequences; it may
 *   be the final_state of an earlier call (but not alias this call's).
 *   cu_seqlens (NULL: none): device pointer to nseq + 1 int64 offsets,
 *   8-byte aligned; batch must be 1, and sequence s is tokens cu_seqlens[s]
 *   .. cu_seqlens[s+1]-1 of batch row 0, scanned on its own from its own
 *   initial state; final_state is then [nseq, dim, dstate].  The offsets
 *   should start at 0, not decrease and end at L; they are not checked
 *   (values read on the device are clamped into [0, L]).  A sequence is
 *   never cut, so L * dim elements must fit 2^31 bytes (else UNSUPPORTED).
 *   Everything else as ssm_scan_fwd, whose call is this one with NULL,
 *   NULL, 0. */
ssm_status_t ssm_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias, int softplus_flag,
                             const float* initial_state, const int64_t* cu_seqlens, int64_t nseq,
                             void* y, float* final_state,
                             int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace for ssm_scan_trap_fwd: that of ssm_scan_fwd_ex_workspace_size
 * for the same arguments plus C_t . B_t of every token (about batch * L * 4
 * bytes).  Returns 0 for arguments the call would reject. */
size_t ssm_scan_trap_fwd_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate, int64_t nseq,
                                        ssm_dtype_t dt);

/* ssm_scan_fwd_ex with the trapezoidal three-term recurrence of Mamba-3
 * ("The State That Must Remember Everything", Part 7, "Mamba-3 (2026)",
 * item 1), which brings in the previous token's input as well:
 *     h_t = alpha_t h_{t-1} + beta_t B_{t-1} u_{t-1} + gamma_t B_t u_t,
 * read as the trapezoidal rule on the step's input integral (the page calls
 * the recurrence a trapezoidal variant of exponential-Euler and leaves the
 * coefficients open):
 *     alpha_t = exp(delta_t A),  beta_t = delta_t/2 * exp(delta_t A),
 *     gamma_t = delta_t/2,
 * with delta_t = softplus(delta_raw + bias) (or raw + bias) as in
 * ssm_scan_fwd.  The readout, D skip and SiLU(z) gate are those of
 * ssm_scan_fwd; final_state is h after the last token.  At the first token of
 * a recurrence (a batch row, or a packed sequence) the previous input is
 * zero, also when an initial state is given: a call starts a sequence, it
 * does not continue one.  Arguments, layouts, ownership and errors as
 * ssm_scan_fwd_ex; the workspace comes from ssm_scan_trap_fwd_workspace_size. */
ssm_status_t ssm_scan_trap_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias, int softplus_flag,
                               const float* initial_state, const int64_t* cu_seqlens, int64_t nseq,
                               void* y, float* final_state,
                               int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The Mamba-2 state-space-duality (SSD) layer ("State Space Models and the
 * Post-Transformer Era", "Mamba-2 and Structured State Space Duality"; "The
 * State That Must Remember Everything", Part 4): every head has one scalar
 * state matrix A (times the identity), which makes the sequence map a causal
 * 1-semiseparable matrix computed blockwise with matrix products.  Per batch
 * row and head (headdim channels sharing the step and A; B_t, C_t shared by
 * the heads of a group) the state H (headdim x dstate) runs
 *     H_t = exp(delta_t A) H_{t-1} + delta_t x_t B_t^T,   H_{-1} = initial_state or 0,
 *     y_t = (H_t C_t + D x_t) * SiLU(z_t)   (skip and gate optional),
 * with delta_t = softplus(delta_raw + bias) (or raw + bias when
 * softplus_flag = 0).  With one group this equals ssm_scan_fwd with dim =
 * heads * headdim, A[d][n] = A[head of d] and the head's step on each of its
 * channels.  Groups: the page casts B_t as the keys and C_t as the queries of
 * masked linear attention; as grouped attention shares keys and queries among
 * heads, runs of heads / ngroups consecutive heads share a group's B_t, C_t
 * (head h reads group h / (heads / ngroups)); each group is then the
 * one-group layer over its heads.
 *   x, z, y: [batch, L, heads, headdim]; delta: [batch, L, heads]; B, C:
 *   [batch, L, ngroups, dstate] (all bf16); ngroups >= 1 divides heads (else
 *   INVALID_ARG); A, D, delta_bias: [heads] fp32;
 *   final_state (nullable): [batch, heads, headdim, dstate] fp32.
 *   initial_state (nullable): the same layout, the state before token 0 of
 *   each (row, head), e.g. the final_state of the call over the tokens before
 *   ("Mamba is attention all you really need, part 2", "The relay"); it may
 *   be the same buffer as final_state.
 *   Required: x, delta, A, B, C, y; optional: D, z, delta_bias,
 *   initial_state, final_state.
 *   x, B, C must be 16-byte aligned, delta, z, y 2-byte, the fp32 arrays
 *   4-byte (else INVALID_ARG).  Supported: dt = BF16, headdim = 64 and
 *   dstate = 32, 64 or 128, with (L + 64) * heads * headdim * 2 and
 *   (L + 64) * ngroups * dstate * 2 bytes below 2^31 (else UNSUPPORTED).  Arithmetic: matrix products with
 *   fp32 accumulation and an fp32 state; C B^T takes bf16 operands (exact),
 *   the other products fp16 operands: x and C convert exactly, the decay-
 *   weighted intra-chunk matrix and the state are rounded to fp16 once where
 *   they enter the output, and the inputs' path into the state is an fp16
 *   hi + lo pair (22 significant bits).  So x, C, the state and the
 *   intermediate products must stay below 65504 in magnitude (the fp16
 *   range): beyond it the outputs become inf or NaN (values are not
 *   inspected).  workspace: workspace_bytes >=
 *   ssm_ssd_fwd_workspace_size() bytes of device memory, 256-byte aligned
 *   (may be NULL when that size is 0), overwritten by the call and not to be
 *   shared with a concurrent call.  y must not alias an input. */
ssm_status_t ssm_ssd_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                         const float* D, const void* z, const float* delta_bias, int softplus_flag,
                         const float* initial_state, void* y, float* final_state, int64_t batch, int64_t L,
                         int64_t heads, int64_t headdim, int64_t ngroups, int64_t dstate, ssm_dtype_t dt,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace ssm_ssd_fwd needs: 0 when there are at most as
 * many (batch row, head) units as compute units (or more than 1.5 per CU);
 * otherwise the states handed between the segments of the left-over units
 * (about (batch * heads - 256) * 8 * headdim * dstate * 4 bytes at most) and a
 * few words of flags.  Returns 0 also for arguments the call would reject. */
size_t ssm_ssd_fwd_workspace_size(int64_t batch, int64_t L, int64_t heads, int64_t headdim, int64_t dstate,
                                  ssm_dtype_t dt);

/* One recurrent (decode) step: the same arithmetic as one token of the scan,
 * reading `state` as h_{t-1} and overwriting it in place with h_t
 * ("Mamba: The State Space Models Challenging the Transformer", "What a
 * state space model actually is": each new token is one cheap state update).
 *   Required: state, u, delta, A, B, C, y.  Optional: D, z, delta_bias.
 *   dstate up to 256.  A Mamba-2 (SSD) layer's step is this call with each
 *   head's step and A repeated over its headdim channels (dim = heads *
 *   headdim), continuing the state ssm_ssd_fwd leaves.
 *   state must not alias any other argument. */
ssm_status_t ssm_state_update(float* state, const void* u, const void* delta, const float* A, const void* B,
                              const void* C, const float* D, const void* z, const float* delta_bias,
                              int softplus_flag, void* y, int64_t batch, int64_t dim, int64_t dstate,
                              ssm_dtype_t dt, hipStream_t stream);

/* Bytes of device workspace that ssm_scan_bwd needs for this shape (always
 * > 0 for a valid shape): the packed B/C records, the state entering every
 * 16-token block of every 64-channel tile (about batch * L * dim * dstate *
 * 4 / 16 bytes), and per-tile partial sums of dB and dC (about 2 * batch *
 * L * dim / 64 * dstate * 4 bytes) and of dA, dD and d(delta_bias) per batch
 * row (and per chunk slot, plus the adjoints handed between chunks, when
 * there are between 1 and 1.5 tiles of 64 channels per compute unit).  With
 * nseq > 0 packed sequences (batch 1): partial rows per sequence, a few more
 * checkpoints per sequence and the launch order.  Returns 0 for arguments
 * ssm_scan_bwd would reject. */
size_t ssm_scan_bwd_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate, int64_t nseq,
                                   ssm_dtype_t dt);

/* Backward of ssm_scan_fwd, or of ssm_scan_fwd_ex from initial states and
 * over packed sequences: the gradients of
 *     sum(y * dy) + sum(final_state * dfinal_state)
 * with respect to u, delta, A, B, C, D, z, delta_bias and the initial
 * state, for the same inputs and flags as the forward call.  The states are recomputed from the
 * inputs, not stored by the forward ("Mamba is attention all you really need,
 * part 2", "Keeping the pad on the desk"; "The state that must remember
 * everything", "The Hardware-Aware Way Out", rematerialization).
 *   Inputs as for ssm_scan_fwd, plus dy [batch, L, dim] in dtype dt,
 *   dfinal_state [batch, dim, dstate] fp32 (NULL: no gradient reaches the
 *   final state) and initial_state [batch, dim, dstate] fp32 (NULL: zero).
 *   Outputs, all overwritten: du, ddelta [batch, L, dim], dB, dC [batch, L,
 *   dstate] in dtype dt (gradients of the sequence inputs, rounded like y);
 *   dA [dim, dstate] fp32.  dD [dim], dz [batch, L, dim] (dtype dt) and
 *   ddelta_bias [dim] fp32 are written when both the input (D, z,
 *   delta_bias) and the output pointer are non-NULL; dinitial_state [batch,
 *   dim, dstate] fp32 is written when non-NULL (with or without an initial
 *   state: it is the adjoint reaching h_{-1}).  The gradient of delta
 *   is the one of the raw input (through softplus and the bias when on).
 *   dA, dD and ddelta_bias sum over the batch and the sequence, dB and dC
 *   over the channels, in a fixed order (results are deterministic).
 *   cu_seqlens (NULL: none), nseq: packed sequences as in ssm_scan_fwd_ex
 *   (batch 1, nseq + 1 int64 device offsets, 8-byte aligned, clamped into
 *   [0, L] on the device); each sequence runs from initial_state[s] with
 *   its own final state, so initial_state, dfinal_state and dinitial_state
 *   are then [nseq, dim, dstate], and an empty sequence hands
 *   dfinal_state[s] to dinitial_state[s] unchanged.
 *   No output may alias an input or another output.  workspace must hold
 *   ssm_scan_bwd_workspace_size() bytes of device memory, 256-byte aligned.
 *   UNSUPPORTED for dstate > 64 or batch > 65535, and where a tile's dB/dC
 *   partial row ((L + 128) * dstate * 4 bytes, dstate rounded up to the
 *   kernel's state count) or, above 32 states, an fp32 row of L * dim
 *   partials reaches 2^31 bytes.  Above 32 states the states are taken in two
 *   halves, the first leaving its per-(token, channel) partial sums in the
 *   workspace (3 * batch * L * dim * 4 more bytes). */
ssm_status_t ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                          const float* D, const void* z, const float* delta_bias, int softplus_flag,
                          const void* dy, const float* dfinal_state, const float* initial_state,
                          const int64_t* cu_seqlens, int64_t nseq,
                          void* du, void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                          float* ddelta_bias, float* dinitial_state,
                          int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace that ssm_scan_trap_bwd needs (arguments as
 * ssm_scan_bwd_workspace_size; there is no chained plan, so no carried
 * adjoints).  Returns 0 for arguments ssm_scan_trap_bwd would reject. */
size_t ssm_scan_trap_bwd_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate, int64_t nseq,
                                        ssm_dtype_t dt);

/* Backward of ssm_scan_trap_fwd: the gradients of
 *     sum(y * dy) + sum(final_state * dfinal_state)
 * for Mamba-3's trapezoidal three-term recurrence ("The State That Must
 * Remember Everything", Part 7, "Mamba-3 (2026)", item 1) with the
 * coefficients ssm_scan_trap_fwd uses (alpha_t = exp(delta_t A), beta_t =
 * delta_t/2 alpha_t, gamma_t = delta_t/2, no previous input at the first
 * token of a batch row or packed sequence).  The states are recomputed from
 * checkpoints of the same recurrence, not stored by the forward.  Arguments,
 * outputs, layouts, packed sequences, dstate range and errors as
 * ssm_scan_bwd; the workspace must hold ssm_scan_trap_bwd_workspace_size()
 * bytes.  Every tile of 64 channels runs in one workgroup (no chained
 * plan). */
ssm_status_t ssm_scan_trap_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias, int softplus_flag,
                               const void* dy, const float* dfinal_state, const float* initial_state,
                               const int64_t* cu_seqlens, int64_t nseq,
                               void* du, void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                               float* ddelta_bias, float* dinitial_state,
                               int64_t batch, int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Outcome of the kernels of the last call that used `workspace` (any entry
 * point taking a workspace): SSM_OK, or SSM_ERR_HANDOFF_TIMEOUT when a chained
 * hand-off wait of that call ran out (its dependent outputs are then NaN).
 * Enqueues a 4-byte device-to-host copy of the workspace's status word on
 * `stream` and synchronises the stream, so it returns after the call's
 * kernels.  workspace NULL or workspace_bytes 0 (an SSD call that needed no
 * workspace): SSM_OK.  A workspace below 16 bytes or not 256-byte aligned:
 * SSM_ERR_INVALID_ARG; a failed copy: SSM_ERR_HIP.  Meaningless for a
 * workspace no call has used yet. */
ssm_status_t ssm_workspace_status(const void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char* ssm_status_string(ssm_status_t s);

#ifdef __cplusplus
}
#endif
#endif /* SSM_SCAN_H */
