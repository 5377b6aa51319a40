// scan_bf16_chained.hip -- scan_kernel instantiations: bf16 storage, kModeChained.
#define SSM_IO BF16
#define SSM_MODE kModeChained
#define SSM_RULE kRuleEuler
#include "scan_launch.inc"
