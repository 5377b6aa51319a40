// scan_f32_chained_trap.hip -- scan_kernel instantiations: f32 storage, kModeChained, trapezoidal rule.
#define SSM_IO F32
#define SSM_MODE kModeChained
#define SSM_RULE kRuleTrap
#include "scan_launch.inc"
