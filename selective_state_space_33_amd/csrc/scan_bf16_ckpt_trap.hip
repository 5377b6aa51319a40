// scan_bf16_ckpt_trap.hip -- scan_kernel instantiations: bf16 storage, kModeCkpt, trapezoidal rule.
#define SSM_IO BF16
#define SSM_MODE kModeCkpt
#define SSM_RULE kRuleTrap
#include "scan_launch.inc"
