// scan_bf16_agg_trap.hip -- scan_kernel instantiations: bf16 storage, kModeAgg, trapezoidal rule.
#define SSM_IO BF16
#define SSM_MODE kModeAgg
#define SSM_RULE kRuleTrap
#include "scan_launch.inc"
