// scan_bf16_chained_trap.hip -- scan_kernel instantiations: bf16 storage, kModeChained, trapezoidal rule.
#define SSM_IO BF16
#define SSM_MODE kModeChained
#define SSM_RULE kRuleTrap
#include "scan_launch.inc"
