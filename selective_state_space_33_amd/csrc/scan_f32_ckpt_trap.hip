// scan_f32_ckpt_trap.hip -- scan_kernel instantiations: f32 storage, kModeCkpt, trapezoidal rule.
#define SSM_IO F32
#define SSM_MODE kModeCkpt
#define SSM_RULE kRuleTrap
#include "scan_launch.inc"
