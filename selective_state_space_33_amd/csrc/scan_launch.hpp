// scan_launch.hpp -- launch of scan_kernel for a runtime-chosen variant.
//
// The kernel is instantiated per storage type, launch mode and discretisation
// rule in separate translation units (scan_<type>_<mode>[_trap].hip), which
// are compiled in parallel; ssm_scan.hip only calls launch_scan.
#pragma once

#include <hip/hip_runtime.h>

#include "scan_kernels.hpp"

namespace ssm {

// (npl, G): states per lane and wavefronts; vw: prologue width (the
// variant's preferred width, else 1); tb: tokens per block (16, or 32 where
// variant_has_tb32).  Returns hipErrorInvalidValue for a variant that does
// not exist.
template <class IO, int MODE, int RULE = kRuleEuler>
hipError_t launch_scan(int npl, int G, int vw, int tb, const ScanParams& p, dim3 grid, hipStream_t s);

// Instantiated (each in its own translation unit) for these eighteen combinations.
extern template hipError_t launch_scan<F32, kModeFull>(int, int, int, int, const ScanParams&, dim3, hipStream_t);
extern template hipError_t launch_scan<F32, kModeAgg>(int, int, int, int, const ScanParams&, dim3, hipStream_t);
extern template hipError_t launch_scan<F32, kModeChained>(int, int, int, int, const ScanParams&, dim3, hipStream_t);
extern template hipError_t launch_scan<BF16, kModeFull>(int, int, int, int, const ScanParams&, dim3, hipStream_t);
extern template hipError_t launch_scan<BF16, kModeAgg>(int, int, int, int, const ScanParams&, dim3, hipStream_t);
extern template hipError_t launch_scan<F32, kModeCkpt>(int, int, int, int, const ScanParams&, dim3, hipStream_t);
extern template hipError_t launch_scan<BF16, kModeCkpt>(int, int, int, int, const ScanParams&, dim3, hipStream_t);
extern template hipError_t launch_scan<F32, kModeChainedCkpt>(int, int, int, int, const ScanParams&, dim3,
                                                             hipStream_t);
extern template hipError_t launch_scan<BF16, kModeChainedCkpt>(int, int, int, int, const ScanParams&, dim3,
                                                              hipStream_t);
extern template hipError_t launch_scan<BF16, kModeChained>(int, int, int, int, const ScanParams&,
                                                           dim3, hipStream_t);
extern template hipError_t launch_scan<F32, kModeFull, kRuleTrap>(int, int, int, int, const ScanParams&, dim3,
                                                                 hipStream_t);
extern template hipError_t launch_scan<F32, kModeAgg, kRuleTrap>(int, int, int, int, const ScanParams&, dim3,
                                                                hipStream_t);
extern template hipError_t launch_scan<F32, kModeChained, kRuleTrap>(int, int, int, int, const ScanParams&, dim3,
                                                                    hipStream_t);
extern template hipError_t launch_scan<BF16, kModeFull, kRuleTrap>(int, int, int, int, const ScanParams&, dim3,
                                                                  hipStream_t);
extern template hipError_t launch_scan<BF16, kModeAgg, kRuleTrap>(int, int, int, int, const ScanParams&, dim3,
                                                                 hipStream_t);
extern template hipError_t launch_scan<BF16, kModeChained, kRuleTrap>(int, int, int, int, const ScanParams&, dim3,
                                                                     hipStream_t);
extern template hipError_t launch_scan<F32, kModeCkpt, kRuleTrap>(int, int, int, int, const ScanParams&, dim3,
                                                                 hipStream_t);
extern template hipError_t launch_scan<BF16, kModeCkpt, kRuleTrap>(int, int, int, int, const ScanParams&, dim3,
                                                                  hipStream_t);

// Variants (states per lane, wavefronts).  Each exists with its preferred
// prologue width (channels per thread: 4 up to 4 wavefronts, 2 for 8, 1 for
// 16) and with width 1.
inline bool variant_exists(int npl, int G) {
  if (npl == 4 && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16)) return true;
  return (npl == 2 && G == 8) || (npl == 1 && G == 16) || (npl == 8 && G == 2) || (npl == 16 && G == 1);
}
inline int preferred_vw(int G) { return G <= 4 ? 4 : (G == 8 ? 2 : 1); }
// 32-token blocks exist for (2, 8) at its preferred width, outside the chunk-pair pass.
inline bool variant_has_tb32(int npl, int G, int vw, int mode) {
  return npl == 2 && G == 8 && vw == 2 && (mode == kModeFull || mode == kModeChained);
}

}  // namespace ssm
