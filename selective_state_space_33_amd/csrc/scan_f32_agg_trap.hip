// scan_f32_agg_trap.hip -- scan_kernel instantiations: f32 storage, kModeAgg, trapezoidal rule.
#define SSM_IO F32
#define SSM_MODE kModeAgg
#define SSM_RULE kRuleTrap
#include "scan_launch.inc"
