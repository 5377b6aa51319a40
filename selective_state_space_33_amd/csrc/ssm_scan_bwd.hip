// ssm_scan_bwd.hip -- C-ABI entry points of the selective scan backward pass
// (declared with their contracts in include/ssm_scan.h).
//
// One call: pack B/C into the forward's records; a forward launch in
// checkpoint mode leaves the state entering every 16-token block of every
// tile; the backward kernel walks each tile's blocks from the last to the
// first, recomputing the states it needs (one workgroup per tile, or, with
// between 1 and 1.5 tiles per CU, one per CU with the left-over tiles' chunks
// chained in); two small kernels add the partial sums over tiles (dB, dC)
// and batch rows and chunk slots (dA, dD, dbias) in a fixed order.
//
// SSM_BWD_CHAINED=0 (environment) keeps one workgroup per tile; for tests and
// timing comparisons.
#include "ssm_scan.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "bwd_kernels.hpp"
#include "host_common.hpp"
#include "order_kernel.hpp"
#include "scan_launch.hpp"

namespace ssm {
namespace {

constexpr int64_t kBwdMaxBatch = 65535;
constexpr int64_t kBwdMaxState = 64;
constexpr int64_t kBwdOneLaunchState = 32;  // states one backward launch covers (4 per lane, 8 wavefronts)
constexpr int64_t kBwdMaxChained = 8;  // chunks per left-over tile (the hand-offs run in series)
constexpr int64_t kBwdMinChunk = 256;   // tokens: the checkpoint pass never cuts the sequence finer

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
bool is_aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Variant: 2 states per lane over 8 wavefronts up to 16 states, 4 per lane up to 32;
// above 32 (wide states, up to 64) two launches of the 4-per-lane kernel, one
// per half of the states, over records and checkpoints laid out for 16 groups
// of 4 (the checkpoint pass runs the forward's 16-wavefront variant).
// Chained plan (CUs < T <= 1.5 CUs): n_long = CUs whole tiles, the r = T - CUs
// others in Ks = CUs / r chunks of blocks (at most 8); the checkpoint pass is
// chained the same way, as the forward plans it: Kc = CUs / r chunks, at most
// 8 and no shorter than 256 tokens, in whole trips of its loop.
struct BwdPlan {
  int npl, G;
  int g_total;   // state groups of the records and checkpoints (G, or 2G for wide states)
  bool wide;
  int64_t nseq;  // packed sequences of batch row 0 (0: none)
  int64_t Lp, ntd, T, ckpt_blocks;
  int n_long, n_split, Ks, chunk_blocks;
  // the checkpoint pass, chained alike: Kc chunks of ck_len tokens per left-over tile
  int Kc;
  int64_t ck_len;
};

// Packed sequences (nseq > 0, batch 1): one unit per (tile column, sequence),
// no chained plan; each sequence's checkpoints start kPackedCkptSlack blocks
// further per sequence before it, so a tile column holds Lp / 16 +
// kPackedCkptSlack * nseq of them.
BwdPlan plan_bwd(int64_t batch, int64_t L, int64_t dim, int64_t N, int64_t nseq, int rule) {
  BwdPlan pl;
  pl.npl = N <= 16 ? 2 : 4;
  pl.G = 8;
  pl.wide = N > kBwdOneLaunchState;
  pl.g_total = pl.wide ? 2 * pl.G : pl.G;
  pl.nseq = nseq > 0 ? nseq : 0;
  pl.Lp = cdiv(L, kTrip) * kTrip;  // whole trips of the checkpoint launch
  pl.ntd = cdiv(dim, 64);
  pl.T = (pl.nseq > 0 ? pl.nseq : batch) * pl.ntd;
  pl.ckpt_blocks = pl.Lp / kBwdTB + kPackedCkptSlack * pl.nseq;
  pl.n_long = 0;
  pl.n_split = 0;
  pl.Ks = 1;
  pl.chunk_blocks = 0;
  pl.Kc = 1;
  pl.ck_len = 0;
  const char* env = getenv("SSM_BWD_CHAINED");
  // (the trapezoidal rule's backward runs one workgroup per tile: no chained plan)
  const bool chained_ok = !(env && atoi(env) == 0) && pl.nseq == 0 && !pl.wide && rule == kRuleEuler;
  const int64_t kBwdNumCU = device_cu_count();
  if (chained_ok && pl.T > kBwdNumCU && 2 * (pl.T - kBwdNumCU) <= kBwdNumCU) {
    const int64_t r = pl.T - kBwdNumCU;
    int64_t K = kBwdNumCU / r;
    if (K > kBwdMaxChained) K = kBwdMaxChained;
    pl.n_long = static_cast<int>(kBwdNumCU);
    pl.n_split = static_cast<int>(r);
    pl.Ks = static_cast<int>(K);
    pl.chunk_blocks = static_cast<int>(cdiv(cdiv(L, kBwdTB), K));
    // the forward's chained plan for the checkpoints: chunk lengths in whole trips of its loop
    int64_t Kc = kBwdNumCU / r;
    if (Kc > kBwdMaxChained) Kc = kBwdMaxChained;
    if (Kc > cdiv(L, kBwdMinChunk)) Kc = cdiv(L, kBwdMinChunk);
    if (Kc < 1) Kc = 1;
    pl.ck_len = cdiv(cdiv(L, Kc), kTrip) * kTrip;
    pl.Kc = static_cast<int>(cdiv(L, pl.ck_len));
  }
  return pl;
}

// Workspace: [header words (status, the two launches' tickets, ...), ready
// flags of the backward, then of the checkpoint pass][packed B/C]
// [checkpoints][dB, dC partials][dA, dD, dbias partials (Ks slots of batch
// rows, or one per packed sequence)][carried adjoints][carried
// checkpoint-pass states][packed sequences' launch order].
struct BwdLayout {
  size_t words, bc, ckpt, bcpart, apart, dpart, carry, ckcarry, order, part, total;
  int n_words, bwd_words;
};

BwdLayout bwd_layout(const BwdPlan& pl, int64_t batch, int64_t L, int64_t dim) {
  const int64_t npad = static_cast<int64_t>(pl.npl) * pl.g_total;
  const int64_t slots = pl.n_split > 0 ? pl.Ks : 1;
  const int64_t prow = pl.nseq > 0 ? pl.nseq : batch;  // partial rows per slot
  BwdLayout l;
  l.bwd_words = pl.n_split > 0 ? pl.n_split * pl.Ks : 0;
  l.n_words = kHeaderWords + l.bwd_words + (pl.n_split > 0 ? pl.n_split * pl.Kc : 0);
  l.words = al256(static_cast<size_t>(l.n_words) * sizeof(unsigned));
  l.bc = al256(static_cast<size_t>(batch * pl.Lp + kTBMax) * 2 * npad * sizeof(float));
  l.ckpt = al256(static_cast<size_t>(pl.T * pl.ckpt_blocks) * 64 * npad * sizeof(float));
  l.bcpart = al256(static_cast<size_t>(batch * pl.ntd * pl.Lp) * npad * sizeof(float));
  l.apart = al256(static_cast<size_t>(slots * prow * dim) * npad * sizeof(float));
  l.dpart = al256(static_cast<size_t>(slots * prow * dim) * sizeof(float));
  l.carry = al256(static_cast<size_t>(pl.n_split) * pl.Ks * 64 * npad * sizeof(float));
  l.ckcarry = al256(static_cast<size_t>(pl.n_split) * pl.Kc * 64 * npad * sizeof(float));
  l.order = al256(static_cast<size_t>(pl.nseq) * sizeof(int));
  // wide states: the first half's v, sum t_a A and sum dh B per (row, token, channel)
  l.part = pl.wide ? al256(static_cast<size_t>(batch * L * dim) * sizeof(float)) : 0;
  l.total = l.words + l.bc + l.ckpt + 2 * l.bcpart + l.apart + 2 * l.dpart + l.carry + l.ckcarry + l.order +
            3 * l.part;
  return l;
}

// The kernels address a tile's token rows with 32-bit byte offsets from the
// row block's start.
bool rows_fit(int64_t L, int64_t dim, int64_t es) { return L * dim * es < 0x7fffffffLL - kTrip * dim * es; }
// The kernel reaches a tile's dB/dC partial row ([Lp][states] fp32) and, for
// wide states, the fp32 per-(token, channel) partials of a row through buffer
// resources with 32-bit offsets.
bool plan_fits(const BwdPlan& pl, int64_t L, int64_t dim) {
  const int64_t npad = static_cast<int64_t>(pl.npl) * pl.g_total;
  if (pl.Lp * npad * 4 >= 0x7fffffffLL) return false;
  return !pl.wide || rows_fit(L, dim, 4);
}

template <class IO, int RULE>
hipError_t run_bwd(const BwdPlan& pl, const BwdLayout& lay, const void* B, const void* C, float* bc, ScanParams sp,
                   BwdParams bp, void* dB, void* dC, float* dA, float* dD, float* dbias, int vw, hipStream_t s) {
  const int64_t npad = static_cast<int64_t>(pl.npl) * pl.g_total;
  const dim3 pgrid(static_cast<unsigned>(sp.batch * (pl.Lp / kPackT)));
  // the pack also zeroes the header words and the chained launches' flags
  if (pl.npl == 2)
    hipLaunchKernelGGL((pack_bc_kernel<IO, 2>), pgrid, dim3(256), 0, s, B, C, bc, sp.batch, sp.L, pl.Lp, sp.N,
                       pl.G, bp.status, lay.n_words, static_cast<float*>(nullptr));
  else
    hipLaunchKernelGGL((pack_bc_kernel<IO, 4>), pgrid, dim3(256), 0, s, B, C, bc, sp.batch, sp.L, pl.Lp, sp.N,
                       pl.g_total, bp.status, lay.n_words, static_cast<float*>(nullptr));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (pl.nseq > 0) {  // packed sequences, longest first (the units of a sequence run together)
    hipLaunchKernelGGL(packed_order_kernel, dim3(1), dim3(kOrderBins), 0, s, sp.cu, static_cast<int>(pl.nseq), sp.L,
                       const_cast<int*>(sp.order));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (RULE == kRuleEuler) {
    if (pl.n_split > 0)
      e = launch_scan<IO, kModeChainedCkpt>(pl.npl, pl.G, vw, kBwdTB, sp, dim3(static_cast<unsigned>(pl.n_long)), s);
  }
  if (pl.n_split == 0) {
    if (pl.wide)  // the forward's 4-per-lane, 16-wavefront variant covers all 64 states
      e = launch_scan<IO, kModeCkpt, RULE>(pl.npl, pl.g_total, 1, kBwdTB, sp, dim3(static_cast<unsigned>(pl.T)), s);
    else
      e = launch_scan<IO, kModeCkpt, RULE>(pl.npl, pl.G, vw, kBwdTB, sp, dim3(static_cast<unsigned>(pl.T)), s);
  }
  if (e != hipSuccess) return e;
  const dim3 bgrid(static_cast<unsigned>(pl.n_split > 0 ? pl.n_long : pl.T));
  if (pl.wide) {  // one launch per half of the states; the second finishes the per-(token, channel) gradients
    bp.n_base = 0;
    hipLaunchKernelGGL((scan_bwd_kernel<IO, 4, 8, 1, RULE>), bgrid, dim3(512), 0, s, bp);
    bp.n_base = static_cast<int>(kBwdOneLaunchState);
    hipLaunchKernelGGL((scan_bwd_kernel<IO, 4, 8, 2, RULE>), bgrid, dim3(512), 0, s, bp);
  } else if (pl.npl == 2) {
    hipLaunchKernelGGL((scan_bwd_kernel<IO, 2, 8, 0, RULE>), bgrid, dim3(512), 0, s, bp);
  } else {
    hipLaunchKernelGGL((scan_bwd_kernel<IO, 4, 8, 0, RULE>), bgrid, dim3(512), 0, s, bp);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nbc = sp.batch * sp.L * sp.N;
  hipLaunchKernelGGL((bwd_reduce_bc_kernel<IO>), dim3(static_cast<unsigned>(cdiv(nbc, 256))), dim3(256), 0, s,
                     bp.dB_part, bp.dC_part, dB, dC, sp.batch, sp.L, pl.Lp, sp.N, npad, static_cast<int>(pl.ntd));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t npar = sp.dim * sp.N;
  // the partial slots are further rows of the same sums
  const int64_t rows = (pl.nseq > 0 ? pl.nseq : sp.batch) * (pl.n_split > 0 ? pl.Ks : 1);
  hipLaunchKernelGGL(bwd_reduce_param_kernel, dim3(static_cast<unsigned>(cdiv(npar, 256))), dim3(256), 0, s,
                     bp.dA_part, bp.dD_part, bp.dbias_part, dA, dD, dbias, rows, sp.dim, sp.N, npad);
  return hipGetLastError();
}

}  // namespace
}  // namespace ssm

using namespace ssm;

namespace ssm {
namespace {
size_t bwd_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate, int64_t nseq, ssm_dtype_t dt,
                          int rule) {
  if (batch <= 0 || L <= 0 || dim <= 0 || dstate <= 0 || dstate > kBwdMaxState || batch > kBwdMaxBatch) return 0;
  if (dt != SSM_DTYPE_F32 && dt != SSM_DTYPE_BF16) return 0;
  if (nseq > 0 && batch != 1) return 0;
  const int64_t es = dt == SSM_DTYPE_F32 ? 4 : 2;
  if (!rows_fit(L, dim, es)) return 0;
  const BwdPlan pl = plan_bwd(batch, L, dim, dstate, nseq, rule);
  if (!plan_fits(pl, L, dim)) return 0;
  return bwd_layout(pl, batch, L, dim).total;
}
}  // namespace
}  // namespace ssm

extern "C" size_t ssm_scan_bwd_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate, int64_t nseq,
                                               ssm_dtype_t dt) {
  return bwd_workspace_size(batch, L, dim, dstate, nseq, dt, kRuleEuler);
}

extern "C" size_t ssm_scan_trap_bwd_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate,
                                                    int64_t nseq, ssm_dtype_t dt) {
  return bwd_workspace_size(batch, L, dim, dstate, nseq, dt, kRuleTrap);
}

namespace ssm {
namespace {
ssm_status_t scan_bwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const float* delta_bias, int softplus_flag, const void* dy,
                           const float* dfinal_state, const float* initial_state, const int64_t* cu_seqlens,
                           int64_t nseq, void* du, void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                           float* ddelta_bias, float* dinitial_state, int64_t batch, int64_t L, int64_t dim,
                           int64_t dstate, ssm_dtype_t dt, void* workspace, size_t workspace_bytes,
                           hipStream_t stream, int rule) {
  if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC) return SSM_ERR_INVALID_ARG;
  if (batch <= 0 || L <= 0 || dim <= 0 || dstate <= 0) return SSM_ERR_INVALID_ARG;
  if (dt != SSM_DTYPE_F32 && dt != SSM_DTYPE_BF16) return SSM_ERR_INVALID_ARG;
  const size_t es = dt == SSM_DTYPE_F32 ? 4 : 2;
  const void* seq[] = {u, delta, B, C, dy, du, ddelta, dB, dC, z, dz};
  for (const void* q : seq)
    if (q && !is_aligned(q, es)) return SSM_ERR_INVALID_ARG;
  const float* f32s[] = {A, D, delta_bias, dfinal_state, initial_state, dA, dD, ddelta_bias, dinitial_state};
  for (const float* q : f32s)
    if (q && !is_aligned(q, 4)) return SSM_ERR_INVALID_ARG;
  if (cu_seqlens && (!is_aligned(cu_seqlens, 8) || batch != 1 || nseq <= 0)) return SSM_ERR_INVALID_ARG;
  if (dstate > kBwdMaxState || batch > kBwdMaxBatch) return SSM_ERR_UNSUPPORTED;
  if (!rows_fit(L, dim, static_cast<int64_t>(es))) return SSM_ERR_UNSUPPORTED;
  const BwdPlan pl = plan_bwd(batch, L, dim, dstate, cu_seqlens ? nseq : 0, rule);
  if (!plan_fits(pl, L, dim)) return SSM_ERR_UNSUPPORTED;
  if (pl.T > 0x7fffffffLL || batch * (pl.Lp / kPackT) > 0x7fffffffLL || batch * L * dstate / 256 > 0x7fffffffLL)
    return SSM_ERR_UNSUPPORTED;
  const BwdLayout lay = bwd_layout(pl, batch, L, dim);
  if (!workspace || workspace_bytes < lay.total || !is_aligned(workspace, 256)) return SSM_ERR_INVALID_ARG;

  // The checkpoint launch's prologue width: dim % vw == 0 and rows aligned to vw elements.
  int vw_ok = 1;
  for (int v = 4; v >= 2; v /= 2) {
    const size_t vb = es * v;
    if ((dim % v) == 0 && is_aligned(u, vb) && is_aligned(delta, vb)) {
      vw_ok = v;
      break;
    }
  }
  const int vw = preferred_vw(pl.G) <= vw_ok ? preferred_vw(pl.G) : 1;

  unsigned* words = static_cast<unsigned*>(workspace);
  char* ws = static_cast<char*>(workspace) + lay.words;
  float* bc = reinterpret_cast<float*>(ws);
  float* ckpt = reinterpret_cast<float*>(ws + lay.bc);
  float* dB_part = reinterpret_cast<float*>(ws + lay.bc + lay.ckpt);
  float* dC_part = reinterpret_cast<float*>(ws + lay.bc + lay.ckpt + lay.bcpart);
  float* dA_part = reinterpret_cast<float*>(ws + lay.bc + lay.ckpt + 2 * lay.bcpart);
  float* dD_part = reinterpret_cast<float*>(ws + lay.bc + lay.ckpt + 2 * lay.bcpart + lay.apart);
  float* dbias_part = reinterpret_cast<float*>(ws + lay.bc + lay.ckpt + 2 * lay.bcpart + lay.apart + lay.dpart);
  char* tail = ws + lay.bc + lay.ckpt + 2 * lay.bcpart + lay.apart + 2 * lay.dpart;
  float* carry = lay.carry ? reinterpret_cast<float*>(tail) : nullptr;
  float* ckcarry = lay.ckcarry ? reinterpret_cast<float*>(tail + lay.carry) : nullptr;
  int* order = lay.order ? reinterpret_cast<int*>(tail + lay.carry + lay.ckcarry) : nullptr;
  float* part = lay.part ? reinterpret_cast<float*>(tail + lay.carry + lay.ckcarry + lay.order) : nullptr;
  const unsigned spin = wait_spin_limit();
  const unsigned* never = wait_override(words);

  ScanParams sp = {};
  sp.u = u;
  sp.delta = delta;
  sp.A = A;
  sp.bias = delta_bias;
  sp.bc = bc;
  sp.batch = batch;
  sp.L = L;
  sp.Lp = pl.Lp;
  sp.dim = dim;
  sp.N = dstate;
  sp.chunk_len = L;
  sp.ntd = static_cast<int>(pl.ntd);
  sp.n_long = static_cast<int>(pl.T);
  sp.Ks = 1;
  sp.softplus = softplus_flag ? 1 : 0;
  sp.ckpt = ckpt;
  sp.ckpt_blocks = pl.ckpt_blocks;
  sp.h0 = initial_state;
  if (pl.nseq > 0) {  // the checkpoint pass over every (tile column, sequence)
    sp.n_long = 0;
    sp.n_split = static_cast<int>(pl.ntd);
    sp.Ks = static_cast<int>(pl.nseq);
    sp.cu = cu_seqlens;
    sp.order = order;
  }
  if (pl.n_split > 0) {  // the checkpoint pass chained like the forward
    sp.n_long = pl.n_long;
    sp.n_split = pl.n_split;
    sp.Ks = pl.Kc;
    sp.chunk_len = pl.ck_len;
    sp.carry = ckcarry;
    sp.flags = words + kHeaderWords + lay.bwd_words;  // [n_split][Kc]
    sp.ticket = words + kWordTicket2;
    sp.status = words + kWordStatus;
    sp.spin_limit = spin;
    sp.wait_override = never;
  }

  BwdParams bp = {};
  bp.u = u;
  bp.delta = delta;
  bp.A = A;
  bp.D = D;
  bp.z = z;
  bp.bias = delta_bias;
  bp.bc = bc;
  bp.ckpt = ckpt;
  bp.dy = dy;
  bp.dfs = dfinal_state;
  bp.dh0 = dinitial_state;
  bp.du = du;
  bp.ddelta = ddelta;
  bp.dz = z ? dz : nullptr;
  bp.dA_part = dA_part;
  bp.dD_part = dD_part;
  bp.dbias_part = dbias_part;
  bp.dB_part = dB_part;
  bp.dC_part = dC_part;
  bp.batch = pl.nseq > 0 ? pl.nseq : batch;  // partial rows of dA, dD, dbias
  bp.n_base = 0;
  bp.g_total = pl.g_total;
  if (part) {
    const size_t pn = lay.part / sizeof(float);
    bp.part_v = part;
    bp.part_s1 = part + pn;
    bp.part_s2 = part + 2 * pn;
  }
  bp.cu = cu_seqlens;
  bp.order = order;
  bp.L = L;
  bp.Lp = pl.Lp;
  bp.dim = dim;
  bp.N = dstate;
  bp.ckpt_blocks = pl.ckpt_blocks;
  bp.ntd = static_cast<int>(pl.ntd);
  bp.softplus = softplus_flag ? 1 : 0;
  bp.n_long = pl.n_long;
  bp.n_split = pl.n_split;
  bp.Ks = pl.Ks;
  bp.chunk_blocks = pl.chunk_blocks;
  bp.carry = carry;
  bp.flags = pl.n_split > 0 ? words + kHeaderWords : nullptr;  // [n_split][Ks]
  bp.ticket = words + kWordTicket;
  bp.status = words + kWordStatus;
  bp.spin_limit = spin;
  bp.wait_override = never;

  float* dD_out = D ? dD : nullptr;
  float* dbias_out = delta_bias ? ddelta_bias : nullptr;
  hipError_t e;
  if (rule == kRuleTrap)
    e = dt == SSM_DTYPE_F32
            ? run_bwd<F32, kRuleTrap>(pl, lay, B, C, bc, sp, bp, dB, dC, dA, dD_out, dbias_out, vw, stream)
            : run_bwd<BF16, kRuleTrap>(pl, lay, B, C, bc, sp, bp, dB, dC, dA, dD_out, dbias_out, vw, stream);
  else
    e = dt == SSM_DTYPE_F32
            ? run_bwd<F32, kRuleEuler>(pl, lay, B, C, bc, sp, bp, dB, dC, dA, dD_out, dbias_out, vw, stream)
            : run_bwd<BF16, kRuleEuler>(pl, lay, B, C, bc, sp, bp, dB, dC, dA, dD_out, dbias_out, vw, stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}
}  // namespace
}  // namespace ssm

extern "C" ssm_status_t ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                     const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                     const void* dy, const float* dfinal_state, const float* initial_state,
                                     const int64_t* cu_seqlens, int64_t nseq, void* du,
                                     void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                                     float* ddelta_bias, float* dinitial_state, int64_t batch,
                                     int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  return scan_bwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus_flag, dy, dfinal_state, initial_state,
                       cu_seqlens, nseq, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, batch, L, dim,
                       dstate, dt, workspace, workspace_bytes, stream, kRuleEuler);
}

extern "C" ssm_status_t ssm_scan_trap_bwd(const void* u, const void* delta, const float* A, const void* B,
                                          const void* C, const float* D, const void* z, const float* delta_bias,
                                          int softplus_flag, const void* dy, const float* dfinal_state,
                                          const float* initial_state, const int64_t* cu_seqlens, int64_t nseq,
                                          void* du, void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                                          float* ddelta_bias, float* dinitial_state, int64_t batch, int64_t L,
                                          int64_t dim, int64_t dstate, ssm_dtype_t dt, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  return scan_bwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus_flag, dy, dfinal_state, initial_state,
                       cu_seqlens, nseq, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, batch, L, dim,
                       dstate, dt, workspace, workspace_bytes, stream, kRuleTrap);
}
