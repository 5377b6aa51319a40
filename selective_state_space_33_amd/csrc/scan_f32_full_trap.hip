// scan_f32_full_trap.hip -- scan_kernel instantiations: f32 storage, kModeFull, trapezoidal rule.
#define SSM_IO F32
#define SSM_MODE kModeFull
#define SSM_RULE kRuleTrap
#include "scan_launch.inc"
