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
#include "scan_launch.hpp"

namespace ssm {
namespace {

constexpr int64_t kBwdMaxBatch = 65535;
constexpr int64_t kBwdMaxState = 32;
constexpr int64_t kBwdNumCU = 256;  // MI355X compute units

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
bool is_aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Variant: 2 states per lane over 8 wavefronts up to 16 states, 4 per lane up to 32.
// Chained plan (CUs < T <= 1.5 CUs): n_long = CUs whole tiles, the r = T - CUs
// others in Ks = CUs / r chunks of blocks (at most 8).
struct BwdPlan {
  int npl, G;
  int64_t Lp, ntd, T, ckpt_blocks;
  int n_long, n_split, Ks, chunk_blocks;
  // the checkpoint pass, chained alike: Kc chunks of ck_len tokens per left-over tile
  int Kc;
  int64_t ck_len;
};

BwdPlan plan_bwd(int64_t batch, int64_t L, int64_t dim, int64_t N) {
  BwdPlan pl;
  pl.npl = N <= 16 ? 2 : 4;
  pl.G = 8;
  pl.Lp = cdiv(L, kTrip) * kTrip;  // whole trips of the checkpoint launch
  pl.ntd = cdiv(dim, 64);
  pl.T = batch * pl.ntd;
  pl.ckpt_blocks = pl.Lp / kBwdTB;
  pl.n_long = 0;
  pl.n_split = 0;
  pl.Ks = 1;
  pl.chunk_blocks = 0;
  pl.Kc = 1;
  pl.ck_len = 0;
  const char* env = getenv("SSM_BWD_CHAINED");
  const bool chained_ok = !(env && atoi(env) == 0);
  if (chained_ok && pl.T > kBwdNumCU && 2 * (pl.T - kBwdNumCU) <= kBwdNumCU) {
    const int64_t r = pl.T - kBwdNumCU;
    int64_t K = kBwdNumCU / r;
    if (K > 8) K = 8;
    pl.n_long = static_cast<int>(kBwdNumCU);
    pl.n_split = static_cast<int>(r);
    pl.Ks = static_cast<int>(K);
    pl.chunk_blocks = static_cast<int>(cdiv(cdiv(L, kBwdTB), K));
    // the forward's chained plan for the checkpoints: chunk lengths in whole trips of its loop
    pl.Kc = static_cast<int>(kBwdNumCU / r);
    pl.ck_len = cdiv(cdiv(L, pl.Kc), kTrip) * kTrip;
  }
  return pl;
}

// Workspace: [packed B/C][checkpoints][dB, dC partials][dA, dD, dbias
// partials (Ks slots)][carried adjoints][carried checkpoint-pass states]
// [flags, ticket, status of the backward; the same of the checkpoint pass].
struct BwdLayout {
  size_t bc, ckpt, bcpart, apart, dpart, carry, ckcarry, words, total;
  int n_words, bwd_words;
};

BwdLayout bwd_layout(const BwdPlan& pl, int64_t batch, int64_t dim) {
  const int64_t npad = static_cast<int64_t>(pl.npl) * pl.G;
  const int64_t slots = pl.n_split > 0 ? pl.Ks : 1;
  BwdLayout l;
  l.bc = al256(static_cast<size_t>(batch * pl.Lp + kTBMax) * 2 * npad * sizeof(float));
  l.ckpt = al256(static_cast<size_t>(pl.T * pl.ckpt_blocks) * 64 * npad * sizeof(float));
  l.bcpart = al256(static_cast<size_t>(batch * pl.ntd * pl.Lp) * npad * sizeof(float));
  l.apart = al256(static_cast<size_t>(slots * batch * dim) * npad * sizeof(float));
  l.dpart = al256(static_cast<size_t>(slots * batch * dim) * sizeof(float));
  l.carry = al256(static_cast<size_t>(pl.n_split) * pl.Ks * 64 * npad * sizeof(float));
  l.ckcarry = al256(static_cast<size_t>(pl.n_split) * pl.Kc * 64 * npad * sizeof(float));
  l.bwd_words = pl.n_split > 0 ? pl.n_split * pl.Ks + 2 : 0;
  l.n_words = pl.n_split > 0 ? l.bwd_words + pl.n_split * pl.Kc + 2 : 0;
  l.words = al256(static_cast<size_t>(l.n_words) * sizeof(unsigned));
  l.total = l.bc + l.ckpt + 2 * l.bcpart + l.apart + 2 * l.dpart + l.carry + l.ckcarry + l.words;
  return l;
}

// The kernels address a tile's token rows with 32-bit byte offsets from the
// row block's start.
bool rows_fit(int64_t L, int64_t dim, int64_t es) { return L * dim * es < 0x7fffffffLL - kTrip * dim * es; }

template <class IO>
hipError_t run_bwd(const BwdPlan& pl, const BwdLayout& lay, const void* B, const void* C, float* bc, ScanParams sp,
                   BwdParams bp, void* dB, void* dC, float* dA, float* dD, float* dbias, int vw, hipStream_t s) {
  const int64_t npad = static_cast<int64_t>(pl.npl) * pl.G;
  const dim3 pgrid(static_cast<unsigned>(sp.batch * (pl.Lp / kPackT)));
  // the pack also zeroes the chained launch's flags, ticket and status
  if (pl.npl == 2)
    hipLaunchKernelGGL((pack_bc_kernel<IO, 2>), pgrid, dim3(256), 0, s, B, C, bc, sp.batch, sp.L, pl.Lp, sp.N,
                       pl.G, bp.flags, lay.n_words, static_cast<float*>(nullptr));
  else
    hipLaunchKernelGGL((pack_bc_kernel<IO, 4>), pgrid, dim3(256), 0, s, B, C, bc, sp.batch, sp.L, pl.Lp, sp.N,
                       pl.G, bp.flags, lay.n_words, static_cast<float*>(nullptr));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (pl.n_split > 0)
    e = launch_scan<IO, kModeChainedCkpt>(pl.npl, pl.G, vw, kBwdTB, sp, dim3(static_cast<unsigned>(pl.n_long)), s);
  else
    e = launch_scan<IO, kModeCkpt>(pl.npl, pl.G, vw, kBwdTB, sp, dim3(static_cast<unsigned>(pl.T)), s);
  if (e != hipSuccess) return e;
  const dim3 bgrid(static_cast<unsigned>(pl.n_split > 0 ? pl.n_long : pl.T));
  if (pl.npl == 2)
    hipLaunchKernelGGL((scan_bwd_kernel<IO, 2, 8>), bgrid, dim3(512), 0, s, bp);
  else
    hipLaunchKernelGGL((scan_bwd_kernel<IO, 4, 8>), bgrid, dim3(512), 0, s, bp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nbc = sp.batch * sp.L * sp.N;
  hipLaunchKernelGGL((bwd_reduce_bc_kernel<IO>), dim3(static_cast<unsigned>(cdiv(nbc, 256))), dim3(256), 0, s,
                     bp.dB_part, bp.dC_part, dB, dC, sp.batch, sp.L, pl.Lp, sp.N, npad, static_cast<int>(pl.ntd));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t npar = sp.dim * sp.N;
  // the partial slots are further rows of the same sums
  const int64_t rows = sp.batch * (pl.n_split > 0 ? pl.Ks : 1);
  hipLaunchKernelGGL(bwd_reduce_param_kernel, dim3(static_cast<unsigned>(cdiv(npar, 256))), dim3(256), 0, s,
                     bp.dA_part, bp.dD_part, bp.dbias_part, dA, dD, dbias, rows, sp.dim, sp.N, npad);
  return hipGetLastError();
}

}  // namespace
}  // namespace ssm

using namespace ssm;

extern "C" size_t ssm_scan_bwd_workspace_size(int64_t batch, int64_t L, int64_t dim, int64_t dstate,
                                               ssm_dtype_t dt) {
  if (batch <= 0 || L <= 0 || dim <= 0 || dstate <= 0 || dstate > kBwdMaxState || batch > kBwdMaxBatch) return 0;
  if (dt != SSM_DTYPE_F32 && dt != SSM_DTYPE_BF16) return 0;
  const int64_t es = dt == SSM_DTYPE_F32 ? 4 : 2;
  if (!rows_fit(L, dim, es)) return 0;
  const BwdPlan pl = plan_bwd(batch, L, dim, dstate);
  return bwd_layout(pl, batch, dim).total;
}

extern "C" ssm_status_t ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                     const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                     const void* dy, const float* dfinal_state, const float* initial_state, void* du,
                                     void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                                     float* ddelta_bias, float* dinitial_state, int64_t batch,
                                     int64_t L, int64_t dim, int64_t dstate, ssm_dtype_t dt, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
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
  if (dstate > kBwdMaxState || batch > kBwdMaxBatch) return SSM_ERR_UNSUPPORTED;
  if (!rows_fit(L, dim, static_cast<int64_t>(es))) return SSM_ERR_UNSUPPORTED;
  const BwdPlan pl = plan_bwd(batch, L, dim, dstate);
  if (pl.T > 0x7fffffffLL || batch * (pl.Lp / kPackT) > 0x7fffffffLL || batch * L * dstate / 256 > 0x7fffffffLL)
    return SSM_ERR_UNSUPPORTED;
  const BwdLayout lay = bwd_layout(pl, batch, dim);
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

  char* ws = static_cast<char*>(workspace);
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
  unsigned* words = lay.n_words ? reinterpret_cast<unsigned*>(tail + lay.carry + lay.ckcarry) : nullptr;

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
  if (pl.n_split > 0) {  // the checkpoint pass chained like the forward
    sp.n_long = pl.n_long;
    sp.n_split = pl.n_split;
    sp.Ks = pl.Kc;
    sp.chunk_len = pl.ck_len;
    sp.carry = ckcarry;
    sp.flags = words + lay.bwd_words;
    sp.ticket = sp.flags + static_cast<int64_t>(pl.n_split) * pl.Kc;
    sp.status = sp.ticket + 1;
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
  bp.batch = batch;
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
  bp.flags = words;
  bp.ticket = words ? words + static_cast<int64_t>(pl.n_split) * pl.Ks : nullptr;
  bp.status = words ? bp.ticket + 1 : nullptr;

  float* dD_out = D ? dD : nullptr;
  float* dbias_out = delta_bias ? ddelta_bias : nullptr;
  const hipError_t e =
      dt == SSM_DTYPE_F32
          ? run_bwd<F32>(pl, lay, B, C, bc, sp, bp, dB, dC, dA, dD_out, dbias_out, vw, stream)
          : run_bwd<BF16>(pl, lay, B, C, bc, sp, bp, dB, dC, dA, dD_out, dbias_out, vw, stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}
