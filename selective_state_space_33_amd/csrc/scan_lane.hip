// scan_lane.hip -- lane_scan_kernel instantiations (one channel per lane) and their launch.
#include "lane_kernels.hpp"

namespace ssm {

template <class IO>
hipError_t launch_lane(int ns, bool structured, bool full, const LaneParams& p, hipStream_t s) {
  const int64_t units = static_cast<int64_t>(p.n_tiles) * (full ? p.K : p.K - 1);
  if (units <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((units + kLaneWaves - 1) / kLaneWaves));
  const dim3 block(64 * kLaneWaves);
  const bool gate = full && p.z != nullptr;
#define SSM_LANE_GO(NS_, ST_, FU_, GA_) \
  if (structured == ST_ && full == FU_ && gate == GA_) \
    hipLaunchKernelGGL((lane_scan_kernel<IO, NS_, ST_, FU_, GA_>), grid, block, 0, s, p);
#define SSM_LANE_CASE(NS_)                  \
  if (ns == NS_) {                          \
    SSM_LANE_GO(NS_, true, true, true)      \
    SSM_LANE_GO(NS_, true, true, false)     \
    SSM_LANE_GO(NS_, true, false, false)    \
    SSM_LANE_GO(NS_, false, true, true)     \
    SSM_LANE_GO(NS_, false, true, false)    \
    SSM_LANE_GO(NS_, false, false, false)   \
    return hipGetLastError();               \
  }
  SSM_LANE_CASE(4)
  SSM_LANE_CASE(8)
  SSM_LANE_CASE(16)
#undef SSM_LANE_CASE
#undef SSM_LANE_GO
  return hipErrorInvalidValue;
}

template hipError_t launch_lane<F32>(int, bool, bool, const LaneParams&, hipStream_t);
template hipError_t launch_lane<BF16>(int, bool, bool, const LaneParams&, hipStream_t);

}  // namespace ssm
