// bwd_kernels.hpp -- gfx950 kernels of the selective scan backward pass.
//
// The forward per (batch b, channel d), as ssm_scan_fwd computes it:
//   x_t = delta_raw_t + bias,  Delta_t = softplus(x_t) (or x_t),
//   a_t = exp(Delta_t A),  h_t = a_t h_{t-1} + Delta_t u_t B_t,
//   v_t = C_t . h_t + D u_t,  y_t = v_t SiLU(z_t) (or v_t).
// Its gradients for output gradients dy (and dh_L, reaching the final state):
//   dv_t = dy_t SiLU(z_t),  dz_t = dy_t v_t SiLU'(z_t),
//   dh_t = C_t dv_t + a_{t+1} dh_{t+1}                       (adjoint, in reverse)
//   per state: t_a = dh_t h_{t-1} a_t,  dA += t_a Delta_t,  dB_t += dh_t Delta_t u_t (over d),
//              dC_t += dv_t h_t (over d);
//   dDelta_t = sum_n (t_a A + dh_t B_t u_t),  du_t = Delta_t sum_n dh_t B_t + D dv_t,
//   ddelta_raw_t = dDelta_t softplus'(x_t),  dbias += ddelta_raw_t,  dD += dv_t u_t.
// The intermediate states are recomputed, not stored by the forward ("Mamba
// is attention all you really need, part 2", "Keeping the pad on the desk";
// "The state that must remember everything", "The Hardware-Aware Way Out"):
// a forward launch (scan_kernel, checkpoint mode) leaves only the state
// entering every 16-token block, and the backward kernel rebuilds each
// block's states from it, in registers, just before running the adjoint back
// through the block.
//
// scan_bwd_kernel: one workgroup per tile of 64 channels of one batch row,
// the forward's layout (G wavefronts, wavefront w owning states w*NPL ..,
// one channel per lane, B/C records by DPP row broadcast).  Blocks are taken
// from the last to the first; per block:
//   P  every thread: (Delta, Delta*u) and dv of its (token, channel) elements
//      into LDS; u, Delta, softplus' and dy*SiLU'(z) stay in its registers;
//   F  every wavefront: recompute its states through the block from the
//      checkpoint, keeping h_t and a_t in registers, and its partial readout
//      in LDS;
//   E1 every thread: v_t = the partial readouts summed in a fixed order +
//      D u_t, and dz_t;
//   R  every wavefront: the adjoint back through the block; per token its
//      partial sums over its states of t_a A and dh B (to LDS), and per state
//      the dB, dC partials summed over groups of 4 lanes (DPP) to LDS;
//   E2 every thread: du, ddelta_raw of its elements; the tile's dB, dC
//      partials (the 16 group sums, in order) to the workspace.
// dA, dD and dbias accumulate in registers over the whole sequence.  Partial
// sums over tiles (dB, dC) and over batch rows (dA, dD, dbias) are added in
// a fixed order by bwd_reduce_*; so every result is deterministic.
//
// Chained launches (more tiles than CUs, up to 1.5 per CU): one workgroup per
// CU runs a whole tile, and the r left-over tiles are cut into Ks chunks of
// blocks, spliced into the whole tiles in reverse order of time.  Ticket j
// (the order workgroups start) owns whole tile j and, for j < r * Ks, chunk
// c = Ks-1 - j / r of left-over tile j % r.  The last chunk in time goes first,
// from the gradient reaching the final state; chunk c < Ks-1 starts from the
// adjoint that chunk c+1 (an earlier ticket) leaves after its first token,
// handed on through device-coherent stores and a ready flag, as the forward's
// chained plan hands on states.  A workgroup runs about (Ks-1-c) chunk-lengths
// of its whole tile before it polls for that flag, so nobody idles; the whole
// tile's running sums wait in registers meanwhile.  dA, dD and dbias of a
// chunk go to partial slot c (a whole tile's to slot 0, zeros to the others),
// so the reduction stays a fixed-order sum.
#pragma once

#include <utility>

#include "common.hpp"

namespace ssm {


struct BwdParams {
  const void* u;
  const void* delta;
  const float* A;
  const float* D;      // nullable
  const void* z;       // nullable
  const float* bias;   // nullable
  const float* bc;     // packed B/C records [batch][G][Lp][2*NPL] (as the forward's)
  const float* ckpt;   // state entering every block: [tiles][ckpt_blocks][64][NPL*G]
  const void* dy;
  const float* dfs;    // nullable: gradient reaching the final state [batch][dim][N]
  float* dh0;          // nullable: gradient of the initial state [batch][dim][N]
  void* du;
  void* ddelta;
  void* dz;            // nullable
  float* dA_part;      // [batch][dim][NPL*G]
  float* dD_part;      // [batch][dim]
  float* dbias_part;   // [batch][dim]
  float* dB_part;      // [batch][ntd][Lp][NPL*G]
  float* dC_part;
  int64_t batch, L, Lp, dim, N, ckpt_blocks;
  int ntd;
  int softplus;
  // Chained launches (n_split > 0): tiles 0 .. n_long-1 whole, n_long .. n_long+n_split-1
  // cut into Ks chunks of chunk_blocks blocks; adjoints handed on through carry
  // [n_split][Ks][64][NPL*G] and flags [n_split][Ks] (zeroed by the pack kernel).  The
  // dA/dD/dbias partials then have Ks slots: row slot * batch + b.
  int n_long, n_split, Ks;
  int chunk_blocks;
  // Packed sequences (cu non-null, batch row 0, no chained plan): unit j is tile
  // column j % ntd of sequence order[j / ntd] (index order when order is null),
  // tokens cu[s] .. cu[s+1]-1 (clamped into [0, L]); the final-state and
  // initial-state gradients and the dA/dD/dbias partial rows are per sequence,
  // and the sequence's checkpoints start at block cu[s] / 16 + kPackedCkptSlack * s.
  const int64_t* cu;
  const int* order;
  // States beyond one launch's NPL * G (wide states, up to 2 * NPL * G): the
  // kernel runs twice, on states n_base .. n_base + NPL*G - 1 of a layout of
  // g_total state groups (records, checkpoints and the dA, dB, dC partials are
  // laid out for all of them).  The first launch leaves its readout partial v
  // and its partial sums of t_a A and dh B per (row, token, channel) in
  // part_v, part_s1, part_s2 ([batch][L][dim] fp32); the second adds them to
  // its own and writes du, ddelta_raw and dz.  n_base 0, g_total G otherwise.
  int n_base, g_total;
  float* part_v;
  float* part_s1;
  float* part_s2;
  float* carry;
  unsigned* flags;
  unsigned* ticket;
  unsigned* status;
  unsigned spin_limit;             // polls per wait (poll_ready)
  const unsigned* wait_override;   // test hook: a word no one sets, polled instead of every flag
};

constexpr int kBwdTB = 16;  // tokens per block (the checkpoint spacing)
// A chained chunk waits for the adjoint handed on to it with poll_ready; past
// the limit it sets the status word and goes on from a NaN adjoint, so the
// kernel always ends and the gradients that depend on the lost hand-off show
// the failure.
// vmcnt(0) with expcnt and lgkmcnt left at their maxima (gfx9 s_waitcnt encoding).
constexpr int kBwdWaitVm0 = 0x0F70;

// Sums over each group of 4 lanes of four values at once, left in all four
// lanes of the group: a butterfly of two quad permutations (lane i ^ 1, then
// lane i ^ 2).  Every lane ends with (x0 + x1) + (x2 + x3), the same bits, so
// all four may store it to the same address and no lane needs a branch.  One
// asm block, so the order is fixed: each value's next step comes four
// instructions after its last, past the two wait states a DPP read of a VALU
// result needs; the leading s_nop covers the inputs' own writes.
__device__ __forceinline__ void quad_allsums4(float& a, float& b, float& c, float& d) {
#define SSM_QUAD_STEP(P)                                                          \
  "v_add_f32_dpp %0, %0, %0 quad_perm:" P " row_mask:0xf bank_mask:0xf\n\t"        \
  "v_add_f32_dpp %1, %1, %1 quad_perm:" P " row_mask:0xf bank_mask:0xf\n\t"        \
  "v_add_f32_dpp %2, %2, %2 quad_perm:" P " row_mask:0xf bank_mask:0xf\n\t"        \
  "v_add_f32_dpp %3, %3, %3 quad_perm:" P " row_mask:0xf bank_mask:0xf\n\t"
  asm("s_nop 1\n\t" SSM_QUAD_STEP("[1,0,3,2]") SSM_QUAD_STEP("[2,3,0,1]")
      : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
#undef SSM_QUAD_STEP
}

// WIDE: 0 for all states in one launch; 1 for the first half of wide states
// (partials out), 2 for the second (partials in, finished gradients out).
//
// RULE = kRuleTrap: the backward of the trapezoidal recurrence
//   h_t = alpha_t q_t + (delta_t/2) u_t B_t,  q_t = h_{t-1} + (delta_t/2) u_{t-1} B_{t-1}
// (alpha_t = exp(delta_t A); no previous input at a recurrence's first
// token).  With g_t = C_t dv_t + alpha_{t+1} g_{t+1} the adjoint of h_t:
//   d delta_t = sum_n g_t (A alpha_t q_t + alpha_t (u_{t-1}/2) B_{t-1} + (u_t/2) B_t)
//   dA       += g_t delta_t alpha_t q_t
//   e_t       = (delta_t/2) g_t + (delta_{t+1}/2) alpha_{t+1} g_{t+1}
//   du_t      = sum_n B_t e_t,   dB_t += u_t e_t,   dC_t += dv_t h_t
// The staged pair per token is (delta, u); R forms the whole d delta and du
// partials of its states, since they need the neighbouring tokens.
template <class IO, int NPL, int G, int WIDE = 0, int RULE = kRuleEuler>
__global__ void __launch_bounds__(64 * G) scan_bwd_kernel(BwdParams p) {
  constexpr bool TRAP = RULE == kRuleTrap;
  constexpr int TB = kBwdTB;
  constexpr int NPAD = NPL * G;
  constexpr int RPT = TB / G;               // element rows per thread
  static_assert(TB % G == 0, "element rows");
  constexpr int NRV = TB * 2 * NPL / 16;    // record registers per block
  static_assert((TB * 2 * NPL) % 16 == 0, "records fill whole registers");
  constexpr int ES = __is_same(IO, F32) ? 4 : 2;
  // the decays a_t of a block are kept from the recompute for the adjoint
  // where registers allow (2 states per lane), else recomputed
  constexpr bool KEEP_A = NPL <= 2;

  __shared__ float2 sDU[TB][64];             // (Delta, Delta*u)
  __shared__ float sDV[TB][64];              // dv
  __shared__ float2 sYS[G][TB][64];          // (sum t_a A, sum dh B); the readout partials (.x) too unless SEP
  // Where LDS allows (2 states per lane), the readout partials have an array of
  // their own, so that the adjoint pass may overwrite sYS while v is still being
  // summed: E1 and R then share one phase.
  constexpr bool SEP = NPL <= 2;
  __shared__ float sYP[SEP ? G : 1][SEP ? TB : 1][64];
  // dB, dC partials: one sum per group of 4 lanes, 16 per (token, state), in
  // rows of 20 floats where LDS allows (so that the 16-byte reads of
  // consecutive rows in the reduction below fall on distinct banks)
  constexpr int RROW = NPL <= 2 ? 20 : 16;
  __shared__ float sRB[TB][NPAD][RROW];
  __shared__ float sRC[TB][NPAD][RROW];
  __shared__ float sAcc[2][G][64];
  __shared__ unsigned sWord;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = w * NPL;
  const int nb = p.n_base;                 // first state of this launch
  const int npg = NPL * p.g_total;         // states of the global layouts (records, checkpoints, partials)
  const int64_t dim = p.dim, L = p.L, N = p.N;
  const bool has_z = p.z != nullptr;
  const bool sp_on = p.softplus != 0;
  const int row_bytes = static_cast<int>(dim * ES);
  const int rec_voff = (lane & 15) * 4;
  int nblk = static_cast<int>((L + TB - 1) / TB);  // blocks of the unit's stretch

  // ---- the tile (64 channels of one batch row) the blocks below work on, and
  // the stretch of its row: tokens t_begin .. t_begin+len-1 (the whole row,
  // or a packed sequence); srow indexes the final-state and initial-state
  // gradients and the dA/dD/dbias partial rows (the batch row, or the sequence)
  int tile = 0;
  int64_t b = 0, d0 = 0, d = 0, t_begin = 0, len = L, srow = 0;
  bool dvalid = false;
  float A2[NPL], An[NPL];
  float Dd = 0.0f, bias_d = 0.0f;
  rsrc_t rs_u, rs_d, rs_z, rs_dy, rs_du, rs_dd, rs_dz, rs_bc;
  rsrc_t rs_dbp, rs_dcp;                   // the tile's dB, dC partial rows from the stretch's first token
  rsrc_t rs_pv, rs_ps1, rs_ps2;            // wide states: the per-(token, channel) partial sums
  const float* ckpt_row = p.ckpt;
  auto set_tile = [&](int t, int64_t tb = 0, int64_t tl = -1, int64_t sr = -1, int64_t ckpt_slot0 = 0) {
    tile = t;
    b = t / p.ntd;
    t_begin = tb;
    len = tl < 0 ? L : tl;
    srow = sr < 0 ? b : sr;
    nblk = static_cast<int>((len + TB - 1) / TB);
    d0 = static_cast<int64_t>(t % p.ntd) * 64;
    d = d0 + lane;
    dvalid = d < dim;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int n = nb + n0 + j;
      An[j] = (dvalid && n < N) ? p.A[d * N + n] : 0.0f;
      A2[j] = An[j] * kLog2e;
    }
    Dd = (dvalid && p.D) ? p.D[d] : 0.0f;
    bias_d = (dvalid && p.bias) ? p.bias[d] : 0.0f;
    // Token rows of the tile (channels d0 .. d0+63 of batch row b), through
    // buffer resources: rows past L read as zero and their stores are
    // dropped; lanes past dim are masked at the stores.  The host keeps L
    // rows of the tensor within 2^31 bytes.
    const int64_t base_off = ((b * L + t_begin) * dim + d0) * ES;
    const int64_t bytes = len * row_bytes - d0 * ES;
    auto rs_of = [&](const void* ptr) {
      return make_rsrc(ptr ? static_cast<const char*>(ptr) + base_off : nullptr, ptr ? bytes : 0);
    };
    rs_u = rs_of(p.u);
    rs_d = rs_of(p.delta);
    rs_z = rs_of(p.z);
    rs_dy = rs_of(p.dy);
    rs_du = rs_of(p.du);
    rs_dd = rs_of(p.ddelta);
    rs_dz = rs_of(p.dz);
    const float* bc_row = p.bc + ((b * p.g_total + nb / NPL + w) * p.Lp + t_begin) * (2 * NPL);
    rs_bc = make_rsrc(bc_row, (p.Lp + 32 - t_begin) * 2 * NPL * static_cast<int64_t>(sizeof(float)));
    ckpt_row = p.ckpt + ((static_cast<int64_t>(t) * p.ckpt_blocks + ckpt_slot0) * 64 + lane) * npg + nb + n0;
    const int64_t prow = ((b * p.ntd + t % p.ntd) * p.Lp + t_begin) * npg;  // (the host keeps Lp * npg * 4 < 2^31)
    const int64_t pbytes = (p.Lp - t_begin) * npg * static_cast<int64_t>(sizeof(float));
    rs_dbp = make_rsrc(p.dB_part + prow, pbytes);
    rs_dcp = make_rsrc(p.dC_part + prow, pbytes);
    if constexpr (WIDE != 0) {  // fp32 rows like the tile's token rows (the host keeps L * dim * 4 < 2^31)
      const int64_t fo = (b * L + t_begin) * dim + d0;
      const int64_t fbytes = (len * dim - d0) * static_cast<int64_t>(sizeof(float));
      rs_pv = make_rsrc(p.part_v + fo, fbytes);
      rs_ps1 = make_rsrc(p.part_s1 + fo, fbytes);
      rs_ps2 = make_rsrc(p.part_s2 + fo, fbytes);
    }
  };

  // ---- running sums of the stretch being worked on: the adjoint entering the
  // next block down, dA, and this lane's dD, dbias terms
  float dhn[NPL], dAacc[NPL];
  float accD = 0.0f, accBias = 0.0f;
  float nxt_d = 0.0f;  // trapezoidal rule: the step of the token after the block (zero past the stretch)
  auto start_from_final = [&]() {  // the gradient reaching the tile's final state
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int n = nb + n0 + j;
      dhn[j] = (dvalid && n < N && p.dfs) ? p.dfs[(srow * dim + d) * N + n] : 0.0f;
      dAacc[j] = 0.0f;
    }
    accD = accBias = 0.0f;
    nxt_d = 0.0f;
  };

  // Two-slot pipeline over the blocks (last to first): the loads of block
  // k-1 are in flight while block k computes.  Unrolled by two so each slot
  // keeps fixed registers (no copies, so no early waits on loads in flight).
  // Every vector-memory operation of the loop is unconditional, so that the
  // compiler can count them: loads and stores share one counter, and a wait
  // for block k's data must not wait for the loads of block k-1 issued after
  // them.  (With a load or store under a branch, the count the compiler can
  // prove on every path is too low, and each block waited for the next one's
  // loads.)  Block k-1 may be the one before the stretch: its buffer loads are
  // then out of range or unused, and its checkpoint index is clamped.
  Raw<IO, 1> qu[2][RPT], qd[2][RPT], qz[2][RPT], qg[2][RPT];
  float qrv[2][NRV], qhs[2][NPL];
  // trapezoidal rule: u and B (this lane's states) of the token before the
  // block; before the stretch they read zero (a recurrence's first token has
  // no previous input)
  Raw<IO, 1> qpu[TRAP ? 2 : 1];
  float qpb[TRAP ? 2 : 1][NPL];
  auto load_block = [&](auto slotc, int k) __attribute__((always_inline)) {
    constexpr int S = decltype(slotc)::value;
    const int t0 = k * TB;
#pragma unroll
    for (int v = 0; v < NRV; ++v)
      qrv[S][v] = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(rs_bc, rec_voff + t0 * (2 * NPL * 4) + v * 64, 0, 0));
#pragma unroll
    for (int j = 0; j < NPL; ++j)  // every lane has a checkpoint row (see P for lanes past dim)
      qhs[S][j] = ckpt_row[static_cast<int64_t>(k < 0 ? 0 : k) * 64 * npg + j];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int off = (t0 + w + i * G) * row_bytes + lane * ES;
      qu[S][i] = buf_load<IO, 1>(rs_u, off, 0);
      qd[S][i] = buf_load<IO, 1>(rs_d, off, 0);
      qz[S][i] = buf_load<IO, 1>(rs_z, off, 0);
      qg[S][i] = buf_load<IO, 1>(rs_dy, off, 0);
    }
    if constexpr (TRAP) {
      qpu[S] = buf_load<IO, 1>(rs_u, (t0 - 1) * row_bytes + lane * ES, 0);
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        qpb[S][j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_bc, ((t0 - 1) * 2 * NPL + j) * 4, 0, 0));
    }
  };
  auto process_block = [&](auto slotc, int k) __attribute__((always_inline)) {
    constexpr int S = decltype(slotc)::value;
    const int t0 = k * TB;
    const float* rv = qrv[S];
    const float* hst = qhs[S];

    // ---- P: elements (row, lane) of the block
    float eu[RPT], edl[RPT], esx[RPT], edv[RPT], egz[RPT];
    bool elive[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = w + i * G;
      // lanes past dim read the next row (and their checkpoints hold whatever the checkpoint pass scanned
      // there): a zero step and dv make every term they add to the dB, dC sums zero, and their own
      // outputs are not stored
      const bool live = t0 + row < len && dvalid;
      float uf, df, zf, gf;
      unpack<IO, 1>(qu[S][i], &uf);
      unpack<IO, 1>(qd[S][i], &df);
      unpack<IO, 1>(qz[S][i], &zf);
      unpack<IO, 1>(qg[S][i], &gf);
      const float x = df + bias_d;
      float dl = sp_on ? __builtin_fmaxf(x, 0.0f) + log1p_exp_neg_abs(x) : x;
      dl = live ? dl : 0.0f;  // padding tokens are identity steps
      // softplus'(x) = sigmoid(x)
      const float sx = sp_on ? __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e)) : 1.0f;
      float g = 1.0f, gp = 0.0f;
      if (has_z) {
        const float sz = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zf * kLog2e));
        g = zf * sz;                                  // SiLU(z)
        gp = sz * __builtin_fmaf(zf, 1.0f - sz, 1.0f);  // SiLU'(z) = s (1 + z (1 - s))
      }
      const float dv = live ? gf * g : 0.0f;
      // (delta, delta*u), or (delta, u) under the trapezoidal rule (u zero past the stretch)
      sDU[row][lane] = make_float2(dl, TRAP ? (live ? uf : 0.0f) : dl * uf);
      sDV[row][lane] = dv;
      eu[i] = uf;
      edl[i] = dl;
      esx[i] = sx;
      edv[i] = dv;
      egz[i] = gf * gp;
      elive[i] = live;
    }
    __syncthreads();

    // ---- F: recompute the block's states from the checkpoint
    float hs[TB][NPL], as[KEEP_A ? TB : 1][NPL];
    float2 kdd[KEEP_A ? TB : 1];  // the block's staged pairs, kept from F for R where registers allow
    float u_before = 0.0f;        // trapezoidal rule: u of the token before the block
    if constexpr (TRAP) unpack<IO, 1>(qpu[S], &u_before);
    {
      float h[NPL];
#pragma unroll
      for (int j = 0; j < NPL; ++j) h[j] = hst[j];
      float up = u_before;  // trapezoidal rule: the previous token's u
      [&]<int... T>(std::integer_sequence<int, T...>) {
        (([&] {
           constexpr int t = T;
           const float2 dd = sDU[t][lane];
           if constexpr (KEEP_A) kdd[t] = dd;
           float yp = 0.0f;
           [&]<int... J>(std::integer_sequence<int, J...>) {
             (([&] {
                constexpr int j = J;
                constexpr int fb = t * 2 * NPL + j, fc = fb + NPL;
                const float a = __builtin_amdgcn_exp2f(dd.x * A2[j]);
                if constexpr (TRAP) {
                  // q = h_{t-1} + (delta_t/2) u_{t-1} B_{t-1};  h_t = alpha q + (delta_t/2) u_t B_t
                  const float w1 = 0.5f * dd.x * up;
                  float q;
                  if constexpr (t > 0) q = fmac_row_bcast<(fb - 2 * NPL) % 16>(h[j], rv[(fb - 2 * NPL) / 16], w1);
                  else q = __builtin_fmaf(w1, qpb[S][j], h[j]);
                  h[j] = __builtin_fmaf(a, q, (0.5f * dd.x * dd.y) * row_bcast<fb % 16>(rv[fb / 16]));
                } else {
                  h[j] = __builtin_fmaf(a, h[j], dd.y * row_bcast<fb % 16>(rv[fb / 16]));
                }
                hs[t][j] = h[j];
                if constexpr (KEEP_A) as[t][j] = a;
                if constexpr (j == 0) yp = row_bcast<fc % 16>(rv[fc / 16]) * h[0];
                else yp = fmac_row_bcast<fc % 16>(yp, rv[fc / 16], h[j]);
              }()),
              ...);
           }(std::make_integer_sequence<int, NPL>{});
           if constexpr (SEP) sYP[w][t][lane] = yp;
           else sYS[w][t][lane].x = yp;
           up = dd.y;
         }()),
         ...);
      }(std::make_integer_sequence<int, TB>{});
    }
    __syncthreads();

    // ---- E1: v and dz of the elements
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = w + i * G;
      float v = SEP ? sYP[0][row][lane] : sYS[0][row][lane].x;
#pragma unroll
      for (int ww = 1; ww < G; ++ww) v += SEP ? sYP[ww][row][lane] : sYS[ww][row][lane].x;
      // fp32 partial of this element in the wide-state arrays (out of range when not live: dropped or zero)
      const int poff = elive[i] ? ((t0 + row) * static_cast<int>(dim) + lane) * 4 : 0x7ffffff0;
      if constexpr (WIDE == 1) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs_pv, poff, 0, 0);  // the other half finishes v
        continue;
      }
      if constexpr (WIDE == 2) v += __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_pv, poff, 0, 0));
      v = __builtin_fmaf(Dd, eu[i], v);
      // without z the store's resource has no range (dropped) and egz is zero
      const float dzv = egz[i] * v;
      const int off = elive[i] ? (t0 + row) * row_bytes + lane * ES : 0x7ffffff0;
      buf_store<IO, 1>(rs_dz, off, 0, &dzv);
    }
    if constexpr (!SEP) __syncthreads();  // R overwrites the partials just read

    // ---- R: the adjoint back through the block
    [&]<int... T>(std::integer_sequence<int, T...>) {
      (([&] {
         constexpr int t = TB - 1 - T;
         const float dv = sDV[t][lane];
         float2 dd;
         if constexpr (KEEP_A) dd = kdd[t];
         else dd = sDU[t][lane];
         float s1 = 0.0f, s2 = 0.0f;
         float pb[NPL], pc[NPL];
         // trapezoidal rule: u of the token before, the step of the token after
         float up = 0.0f, dn = 0.0f, s3 = 0.0f, s5 = 0.0f;
         if constexpr (TRAP) {
           if constexpr (t > 0) up = KEEP_A ? kdd[t - 1].y : sDU[t - 1][lane].y;
           else up = u_before;
           if constexpr (t + 1 < TB) dn = KEEP_A ? kdd[t + 1].x : sDU[t + 1][lane].x;
           else dn = nxt_d;
         }
         static_assert(NPL % 2 == 0, "row sums go four values at a time");
         [&]<int... J>(std::integer_sequence<int, J...>) {
           (([&] {
              constexpr int j = J;
              constexpr int fb = t * 2 * NPL + j, fc = fb + NPL;
              // dh = C dv + dhn and s2 += dh B with the records broadcast in the FMA itself
              const float dh = fmac_row_bcast<fc % 16>(dhn[j], rv[fc / 16], dv);
              float hp;
              if constexpr (t > 0) hp = hs[t - 1][j];
              else hp = hst[j];
              float a;
              if constexpr (KEEP_A) a = as[t][j];
              else a = __builtin_amdgcn_exp2f(dd.x * A2[j]);
              if constexpr (TRAP) {
                // dh is g_t; dhn[j] still holds alpha_{t+1} g_{t+1}
                constexpr int fp = fb - 2 * NPL;  // B_{t-1} within the block's records (t > 0)
                const float w1 = 0.5f * dd.x * up;
                float q;
                if constexpr (t > 0) q = fmac_row_bcast<fp % 16>(hp, rv[fp / 16], w1);
                else q = __builtin_fmaf(w1, qpb[S][j], hp);
                const float ga = dh * a;
                const float ta = ga * q;
                s1 = __builtin_fmaf(ta, An[j], s1);
                dAacc[j] = __builtin_fmaf(ta, dd.x, dAacc[j]);
                if constexpr (t > 0) s3 = fmac_row_bcast<fp % 16>(s3, rv[fp / 16], ga);
                else s3 = __builtin_fmaf(ga, qpb[S][j], s3);
                s2 = fmac_row_bcast<fb % 16>(s2, rv[fb / 16], dh);
                s5 = fmac_row_bcast<fb % 16>(s5, rv[fb / 16], dhn[j]);
                pb[j] = __builtin_fmaf(0.5f * dn * dd.y, dhn[j], (0.5f * dd.x * dd.y) * dh);
                pc[j] = dv * hs[t][j];
                dhn[j] = ga;
              } else {
                const float ta = dh * hp * a;
                s1 = __builtin_fmaf(ta, An[j], s1);
                s2 = fmac_row_bcast<fb % 16>(s2, rv[fb / 16], dh);
                dAacc[j] = __builtin_fmaf(ta, dd.x, dAacc[j]);
                pb[j] = dh * dd.y;
                pc[j] = dv * hs[t][j];
                dhn[j] = a * dh;
              }
            }()),
            ...);
         }(std::make_integer_sequence<int, NPL>{});
#pragma unroll
         for (int j = 0; j < NPL; j += 2) quad_allsums4(pb[j], pb[j + 1], pc[j], pc[j + 1]);
         // the four lanes of a group store the same sum to the same word: no
         // branch, so the block's adjoint steps stay one straight run that the
         // compiler can schedule across (its LDS reads issued early)
#pragma unroll
         for (int j = 0; j < NPL; ++j) {
           sRB[t][n0 + j][lane >> 2] = pb[j];
           sRC[t][n0 + j][lane >> 2] = pc[j];
         }
         if constexpr (TRAP)  // this wavefront's parts of d delta_t and du_t
           sYS[w][t][lane] = make_float2(s1 + 0.5f * (up * s3 + dd.y * s2), 0.5f * (dd.x * s2 + dn * s5));
         else
           sYS[w][t][lane] = make_float2(s1, s2);
       }()),
       ...);
    }(std::make_integer_sequence<int, TB>{});
    if constexpr (TRAP) nxt_d = KEEP_A ? kdd[0].x : sDU[0][lane].x;  // for the block before this one
    __syncthreads();

    // ---- E2: du, ddelta_raw of the elements; the tile's dB, dC partials
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = w + i * G;
      float S1 = sYS[0][row][lane].x, S2 = sYS[0][row][lane].y;
#pragma unroll
      for (int ww = 1; ww < G; ++ww) {
        S1 += sYS[ww][row][lane].x;
        S2 += sYS[ww][row][lane].y;
      }
      const int poff = elive[i] ? ((t0 + row) * static_cast<int>(dim) + lane) * 4 : 0x7ffffff0;
      if constexpr (WIDE == 1) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S1), rs_ps1, poff, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S2), rs_ps2, poff, 0, 0);
        continue;
      }
      if constexpr (WIDE == 2) {
        S1 += __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_ps1, poff, 0, 0));
        S2 += __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_ps2, poff, 0, 0));
      }
      // two-term rule: d delta = sum t_a A + u sum dh B, du = delta sum dh B + D dv;
      // trapezoidal rule: R summed the whole parts
      const float dDelta = TRAP ? S1 : __builtin_fmaf(eu[i], S2, S1);
      const float duv = TRAP ? __builtin_fmaf(Dd, edv[i], S2) : __builtin_fmaf(edl[i], S2, Dd * edv[i]);
      const float ddr = dDelta * esx[i];
      const int off = elive[i] ? (t0 + row) * row_bytes + lane * ES : 0x7ffffff0;
      buf_store<IO, 1>(rs_du, off, 0, &duv);
      buf_store<IO, 1>(rs_dd, off, 0, &ddr);
      if (elive[i]) {
        accD = __builtin_fmaf(edv[i], eu[i], accD);
        accBias += ddr;
      }
    }
    // (token, state) items of the block's dB, dC partials, a fixed number per
    // thread; a token past the stretch (the next packed sequence's) stores out
    // of range.  TB * NPAD is a multiple of 64, so `inb` is wave-uniform.
    constexpr int NITEMS = TB * NPAD, NTH = 64 * G;
#pragma unroll
    for (int it = 0; it < (NITEMS + NTH - 1) / NTH; ++it) {
      const int q = tid + it * NTH;
      const bool inb = q < NITEMS;
      const int t = inb ? q / NPAD : 0, n = inb ? q % NPAD : 0;
      float sb = 0.0f, sc = 0.0f;
      if (inb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sb += sRB[t][n][r];
          sc += sRC[t][n][r];
        }
      }
      const int o = (inb && t0 + t < len) ? ((t0 + t) * npg + nb + n) * 4 : 0x7ffffff0;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sb), rs_dbp, o, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rs_dcp, o, 0, 0);
    }
    // No barrier here: the next block's P writes only sDU and sDV, whose last
    // readers (R) finished at the barrier before E2, and its F writes the
    // partials only after the barrier that follows P.
  };

  // Blocks ke-1 down to kb.  With a stop flag, the run also ends after a pair
  // of blocks once at least k_stop blocks are done and the flag is set
  // (thread 0 polls it, the workgroup reads it through LDS); returns the end
  // of what is left, [kb, returned).
  // POLL (a run with a stop flag): every thread loads the flag once per pair
  // of blocks, unconditionally, and thread 0's value decides; runs without a
  // flag issue no load at all (an unused load would still be waited for
  // before its register is reused).  This lambda and the two above are always
  // inlined: as a called function a block would take the buffer descriptors in
  // vector registers (a loop per access) and a stack frame.
  auto run_blocks = [&](auto pollc, int kb, int ke, const unsigned* stop_flag,
                        int k_stop) __attribute__((always_inline)) -> int {
    constexpr bool POLL = decltype(pollc)::value;
    if (ke <= kb) return kb;
    load_block(IC<0>{}, ke - 1);
    for (int k = ke - 1; k >= kb; k -= 2) {
      unsigned seen = 0u;
      if constexpr (POLL) seen = __hip_atomic_load(stop_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      load_block(IC<1>{}, k - 1);
      process_block(IC<0>{}, k);
      if (k - 1 < kb) break;
      load_block(IC<0>{}, k - 2);
      process_block(IC<1>{}, k - 1);
      if (POLL && ke - (k - 1) >= k_stop && k - 1 > kb) {
        if (tid == 0) sWord = seen;
        __syncthreads();
        const bool stop = sWord != 0u;
        __syncthreads();  // every wavefront has read the word before it is written again
        if (stop) return k - 1;
      }
    }
    return kb;
  };

  // dA, dD, dbias of the current stretch into partial slot `slot`; the other
  // slots of a whole tile are zero.
  auto write_partials = [&](int slot, bool zero_others) {
    const int nslots = p.n_split > 0 ? p.Ks : 1;
    if (dvalid) {
      for (int s = 0; s < nslots; ++s) {
        if (s != slot && !zero_others) continue;
        const int64_t row = static_cast<int64_t>(s) * p.batch + srow;
#pragma unroll
        for (int j = 0; j < NPL; ++j) p.dA_part[(row * dim + d) * npg + nb + n0 + j] = s == slot ? dAacc[j] : 0.0f;
      }
    }
    sAcc[0][w][lane] = accD;
    sAcc[1][w][lane] = accBias;
    __syncthreads();
    if (w == 0 && dvalid) {
      float sd = sAcc[0][0][lane], sb = sAcc[1][0][lane];
#pragma unroll
      for (int ww = 1; ww < G; ++ww) {
        sd += sAcc[0][ww][lane];
        sb += sAcc[1][ww][lane];
      }
      for (int s = 0; s < nslots; ++s) {
        if (s != slot && !zero_others) continue;
        const int64_t row = static_cast<int64_t>(s) * p.batch + srow;
        p.dD_part[row * dim + d] = s == slot ? sd : 0.0f;
        p.dbias_part[row * dim + d] = s == slot ? sb : 0.0f;
      }
    }
    __syncthreads();  // sAcc is free again
  };
  // the adjoint left after token 0 is the gradient of h_{-1}
  auto write_dh0 = [&]() {
    if (dvalid && p.dh0) {
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (nb + n0 + j < N) p.dh0[(srow * dim + d) * N + nb + n0 + j] = dhn[j];
    }
  };

  if (p.cu != nullptr) {  // packed: one workgroup per (tile column, sequence)
    const int col = static_cast<int>(blockIdx.x % p.ntd);
    const int s = p.order ? p.order[blockIdx.x / p.ntd] : static_cast<int>(blockIdx.x / p.ntd);
    int64_t tb = p.cu[s], te = p.cu[s + 1];
    tb = tb < 0 ? 0 : (tb > L ? L : tb);
    te = te < tb ? tb : (te > L ? L : te);
    set_tile(col, tb, te - tb, s, tb / TB + static_cast<int64_t>(kPackedCkptSlack) * s);
    start_from_final();
    run_blocks(IC<false>{}, 0, nblk, nullptr, 0);
    write_dh0();
    write_partials(0, false);
    return;
  }
  if (p.n_split == 0) {  // one workgroup per tile
    set_tile(blockIdx.x);
    start_from_final();
    run_blocks(IC<false>{}, 0, nblk, nullptr, 0);
    write_dh0();
    write_partials(0, false);
    return;
  }

  // ---- chained: whole tile j, and chunk c = Ks-1 - j / n_split of left-over tile j % n_split
  if (tid == 0) sWord = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int j = static_cast<int>(__builtin_amdgcn_readfirstlane(sWord));
  __syncthreads();
  set_tile(j);
  start_from_final();
  if (j >= p.n_split * p.Ks) {
    run_blocks(IC<false>{}, 0, nblk, nullptr, 0);
    write_dh0();
    write_partials(0, true);
    return;
  }
  const int o = j / p.n_split, st = j % p.n_split, c = p.Ks - 1 - o;
  const int kb = c * p.chunk_blocks < nblk ? c * p.chunk_blocks : nblk;
  const int ke = (c + 1) * p.chunk_blocks < nblk ? (c + 1) * p.chunk_blocks : nblk;
  // set once chunk c+1 is done
  const unsigned* my_flag = p.wait_override ? p.wait_override : p.flags + static_cast<int64_t>(st) * p.Ks + c;
  int rest = nblk;
  if (o > 0) rest = run_blocks(IC<true>{}, 0, nblk, my_flag, o * p.chunk_blocks);
  float sdh[NPL], sdA[NPL];
  const float sD = accD, sBias = accBias;
#pragma unroll
  for (int q = 0; q < NPL; ++q) {
    sdh[q] = dhn[q];
    sdA[q] = dAacc[q];
  }
  set_tile(p.n_long + st);
  start_from_final();
  const int64_t crow = (static_cast<int64_t>(st) * p.Ks + c) * 64 + lane;  // carry row [n_split][Ks][64]
  if (o > 0) {
    // the adjoint after chunk c+1: wait for its flag, then read it coherently
    if (tid == 0) {
      const bool ok = poll_ready(my_flag, p.spin_limit);
      if (!ok) __hip_atomic_fetch_or(p.status, kStatusHandoffTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sWord = ok ? 1u : 0u;
    }
    __syncthreads();
    const bool lost = sWord == 0u;  // this wait ran out (not another's)
    __syncthreads();                // read by every wavefront before the word is written again
    if (dvalid) {
#pragma unroll
      for (int q = 0; q < NPL; ++q)
        dhn[q] = lost ? __builtin_nanf("")
                      : __hip_atomic_load(p.carry + crow * NPAD + n0 + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  run_blocks(IC<false>{}, kb, ke, nullptr, 0);
  if (c > 0) {
    if (dvalid) {
#pragma unroll
      for (int q = 0; q < NPL; ++q)
        __hip_atomic_store(p.carry + (crow - 64) * NPAD + n0 + q, dhn[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(kBwdWaitVm0);  // this thread's carry stores have completed
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(p.flags + static_cast<int64_t>(st) * p.Ks + c - 1, 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  } else {
    write_dh0();
  }
  write_partials(c, false);
  // back to the whole tile where it stopped
  set_tile(j);
#pragma unroll
  for (int q = 0; q < NPL; ++q) {
    dhn[q] = sdh[q];
    dAacc[q] = sdA[q];
  }
  accD = sD;
  accBias = sBias;
  run_blocks(IC<false>{}, 0, rest, nullptr, 0);
  write_dh0();
  write_partials(0, true);
}

// dB[b][t][n] (and dC) = sum over the tiles of batch row b of their partials,
// in tile order; rounded to the storage type.
template <class IO>
__global__ void __launch_bounds__(256) bwd_reduce_bc_kernel(const float* __restrict__ dB_part,
                                                           const float* __restrict__ dC_part, void* dB, void* dC,
                                                           int64_t batch, int64_t L, int64_t Lp, int64_t N,
                                                           int64_t npad, int ntd) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= batch * L * N) return;
  const int64_t n = i % N, t = (i / N) % L, b = i / (N * L);
  float sb = 0.0f, sc = 0.0f;
  for (int col = 0; col < ntd; ++col) {
    const int64_t o = ((b * ntd + col) * Lp + t) * npad + n;
    sb += dB_part[o];
    sc += dC_part[o];
  }
  store_vals<IO, 1>(dB, i, &sb);
  store_vals<IO, 1>(dC, i, &sc);
}

// dA[d][n] = sum over batch rows of their partials (and dD[d], dbias[d]), in
// batch order.
__global__ void __launch_bounds__(256) bwd_reduce_param_kernel(const float* __restrict__ dA_part,
                                                              const float* __restrict__ dD_part,
                                                              const float* __restrict__ dbias_part, float* dA,
                                                              float* dD, float* dbias, int64_t batch, int64_t dim,
                                                              int64_t N, int64_t npad) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= dim * N) return;
  const int64_t d = i / N, n = i % N;
  float s = 0.0f;
  for (int64_t b = 0; b < batch; ++b) s += dA_part[(b * dim + d) * npad + n];
  dA[i] = s;
  if (n == 0) {
    float sd = 0.0f, sb = 0.0f;
    for (int64_t b = 0; b < batch; ++b) {
      sd += dD_part[b * dim + d];
      sb += dbias_part[b * dim + d];
    }
    if (dD) dD[d] = sd;
    if (dbias) dbias[d] = sb;
  }
}

}  // namespace ssm
