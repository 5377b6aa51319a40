// ssm_ssd.hip -- C-ABI entry point of the Mamba-2 SSD layer (declared with
// its contract in include/ssm_scan.h): argument checks, then one launch of
// ssd_kernel, one workgroup per (batch row, head).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_kernel.hpp"
#include "ssm_scan.h"

namespace ssm {
namespace {

bool ssd_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

template <int N>
hipError_t launch_ssd(const SsdParams& p, hipStream_t s) {
  hipLaunchKernelGGL((ssd_kernel<N>), dim3(static_cast<unsigned>(p.batch * p.H)), dim3(kSsdThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace ssm

using namespace ssm;

extern "C" ssm_status_t ssm_ssd_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                                    const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                    void* y, float* final_state, int64_t batch, int64_t L, int64_t heads,
                                    int64_t headdim, int64_t dstate, ssm_dtype_t dt, hipStream_t stream) {
  if (!x || !delta || !A || !B || !C || !y) return SSM_ERR_INVALID_ARG;
  if (batch <= 0 || L <= 0 || heads <= 0 || headdim <= 0 || dstate <= 0) return SSM_ERR_INVALID_ARG;
  if (dt != SSM_DTYPE_F32 && dt != SSM_DTYPE_BF16) return SSM_ERR_INVALID_ARG;
  // 16-byte pieces of token rows are loaded; scalars and states are fp32
  if (!ssd_aligned(x, 16) || !ssd_aligned(B, 16) || !ssd_aligned(C, 16) || !ssd_aligned(delta, 2) ||
      !ssd_aligned(y, 2) || (z && !ssd_aligned(z, 2)))
    return SSM_ERR_INVALID_ARG;
  const float* f32s[] = {A, D, delta_bias, final_state};
  for (const float* q : f32s)
    if (q && !ssd_aligned(q, 4)) return SSM_ERR_INVALID_ARG;
  if (dt != SSM_DTYPE_BF16 || headdim != kSsdP || (dstate != 32 && dstate != 64 && dstate != 128))
    return SSM_ERR_UNSUPPORTED;
  // token rows are addressed with 32-bit byte offsets (up to one chunk past L)
  const int64_t rows = L + kSsdQ;
  if (rows * heads * headdim * 2 >= 0x7fffffffLL || rows * dstate * 2 >= 0x7fffffffLL ||
      batch * heads > 0x7fffffffLL)
    return SSM_ERR_UNSUPPORTED;
  SsdParams p;
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
  p.batch = batch;
  p.L = L;
  p.H = heads;
  p.softplus = softplus_flag ? 1 : 0;
  hipError_t e;
  if (dstate == 32)
    e = launch_ssd<32>(p, stream);
  else if (dstate == 64)
    e = launch_ssd<64>(p, stream);
  else
    e = launch_ssd<128>(p, stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}
