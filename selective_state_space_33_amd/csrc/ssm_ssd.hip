// ssm_ssd.hip -- C-ABI entry points of the Mamba-2 SSD layer (declared with
// their contracts in include/ssm_scan.h): argument checks, the plan, then one
// launch of ssd_kernel.
//
// Plan: one workgroup per unit (batch row, head) walks the unit's chunks in
// order.  With between 1 and 1.5 units per CU, one workgroup per CU runs a
// whole unit and the r left-over units are cut into Ks = CUs / r segments of
// the sequence (at most 8), chained: segment s starts from the state segment
// s-1 hands on (carry and flags in the workspace, zeroed first by a small
// kernel).  SSM_SSD_CHAINED=0 (environment) keeps one workgroup per unit, for
// tests and timing comparisons.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "host_common.hpp"
#include "ssd_kernel.hpp"
#include "ssm_scan.h"

namespace ssm {
namespace {

bool ssd_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t ssd_al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace of the chained plan: [header words (status, ticket, ...) and
// ready flags][carried states]; none otherwise.
struct SsdPlan {
  int n_long, n_split, Ks;
  int64_t seg_chunks;
  size_t carry_bytes, word_bytes, total;
  int n_words;
};

SsdPlan plan_ssd(int64_t batch, int64_t L, int64_t heads, int64_t dstate) {
  SsdPlan pl = {};
  pl.Ks = 1;
  const int64_t T = batch * heads;
  const int64_t kSsdNumCU = device_cu_count();
  const char* env = getenv("SSM_SSD_CHAINED");
  const bool chained_ok = !(env && atoi(env) == 0);
  if (chained_ok && T > kSsdNumCU && 2 * (T - kSsdNumCU) <= kSsdNumCU) {
    const int64_t r = T - kSsdNumCU;
    int64_t K = kSsdNumCU / r;
    if (K > 8) K = 8;
    const int64_t nchunks = (L + kSsdQ - 1) / kSsdQ;
    pl.n_long = static_cast<int>(kSsdNumCU);
    pl.n_split = static_cast<int>(r);
    pl.Ks = static_cast<int>(K);
    pl.seg_chunks = (nchunks + K - 1) / K;
    pl.carry_bytes = ssd_al256(static_cast<size_t>(r * K) * kSsdP * dstate * sizeof(float));
    pl.n_words = static_cast<int>(kHeaderWords + r * K);
    pl.word_bytes = ssd_al256(static_cast<size_t>(pl.n_words) * sizeof(unsigned));
  }
  pl.total = pl.carry_bytes + pl.word_bytes;
  return pl;
}

bool ssd_shape_ok(int64_t L, int64_t heads, int64_t headdim, int64_t ngroups, int64_t dstate, ssm_dtype_t dt) {
  if (dt != SSM_DTYPE_BF16 || headdim != kSsdP || (dstate != 32 && dstate != 64 && dstate != 128)) return false;
  // token rows are addressed with 32-bit byte offsets (up to one chunk past L)
  const int64_t rows = L + kSsdQ;
  return rows * heads * headdim * 2 < 0x7fffffffLL && rows * ngroups * dstate * 2 < 0x7fffffffLL;
}

template <int N>
hipError_t launch_ssd(const SsdParams& p, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL((ssd_kernel<N>), dim3(grid), dim3(64 * ssd_waves(N)), 0, s, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace ssm

using namespace ssm;

extern "C" size_t ssm_ssd_fwd_workspace_size(int64_t batch, int64_t L, int64_t heads, int64_t headdim,
                                             int64_t dstate, ssm_dtype_t dt) {
  if (batch <= 0 || L <= 0 || heads <= 0 || headdim <= 0 || dstate <= 0) return 0;
  if (!ssd_shape_ok(L, heads, headdim, 1, dstate, dt) || batch * heads > 0x7fffffffLL) return 0;
  return plan_ssd(batch, L, heads, dstate).total;
}

extern "C" ssm_status_t ssm_ssd_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                                    const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                    const float* initial_state, void* y, float* final_state, int64_t batch,
                                    int64_t L, int64_t heads, int64_t headdim, int64_t ngroups, int64_t dstate,
                                    ssm_dtype_t dt, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!x || !delta || !A || !B || !C || !y) return SSM_ERR_INVALID_ARG;
  if (batch <= 0 || L <= 0 || heads <= 0 || headdim <= 0 || dstate <= 0) return SSM_ERR_INVALID_ARG;
  if (ngroups <= 0 || heads % ngroups != 0) return SSM_ERR_INVALID_ARG;
  if (dt != SSM_DTYPE_F32 && dt != SSM_DTYPE_BF16) return SSM_ERR_INVALID_ARG;
  // 16-byte pieces of token rows are loaded; scalars and states are fp32
  if (!ssd_aligned(x, 16) || !ssd_aligned(B, 16) || !ssd_aligned(C, 16) || !ssd_aligned(delta, 2) ||
      !ssd_aligned(y, 2) || (z && !ssd_aligned(z, 2)))
    return SSM_ERR_INVALID_ARG;
  const float* f32s[] = {A, D, delta_bias, final_state, initial_state};
  for (const float* q : f32s)
    if (q && !ssd_aligned(q, 4)) return SSM_ERR_INVALID_ARG;
  if (!ssd_shape_ok(L, heads, headdim, ngroups, dstate, dt) || batch * heads > 0x7fffffffLL)
    return SSM_ERR_UNSUPPORTED;
  const SsdPlan pl = plan_ssd(batch, L, heads, dstate);
  if (pl.total > 0 && (!workspace || workspace_bytes < pl.total || !ssd_aligned(workspace, 256)))
    return SSM_ERR_INVALID_ARG;
  SsdParams p = {};
  p.x = x;
  p.delta = delta;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.z = z;
  p.bias = delta_bias;
  p.y = y;
  p.final_state = final_state;
  p.h0 = initial_state;
  p.batch = batch;
  p.L = L;
  p.H = heads;
  p.ngroups = ngroups;
  p.softplus = softplus_flag ? 1 : 0;
  p.n_long = pl.n_long;
  p.n_split = pl.n_split;
  p.Ks = pl.Ks;
  p.seg_chunks = pl.seg_chunks;
  if (pl.n_split > 0) {
    unsigned* words = static_cast<unsigned*>(workspace);
    p.status = words + kWordStatus;
    p.ticket = words + kWordTicket;
    p.flags = words + kHeaderWords;  // [n_split][Ks]
    p.carry = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.word_bytes);
    p.spin_limit = wait_spin_limit();
    p.wait_override = wait_override(words);
    hipLaunchKernelGGL(ssd_zero_words_kernel, dim3(1), dim3(256), 0, stream, words, pl.n_words);
    const hipError_t ez = hipGetLastError();
    if (ez != hipSuccess) return SSM_ERR_HIP;
  }
  const unsigned grid = static_cast<unsigned>(pl.n_split > 0 ? pl.n_long : batch * heads);
  hipError_t e;
  if (dstate == 32)
    e = launch_ssd<32>(p, grid, stream);
  else if (dstate == 64)
    e = launch_ssd<64>(p, grid, stream);
  else
    e = launch_ssd<128>(p, grid, stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}
