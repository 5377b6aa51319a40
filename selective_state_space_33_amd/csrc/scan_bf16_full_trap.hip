// scan_bf16_full_trap.hip -- scan_kernel instantiations: bf16 storage, kModeFull, trapezoidal rule.
#define SSM_IO BF16
#define SSM_MODE kModeFull
#define SSM_RULE kRuleTrap
#include "scan_launch.inc"
