// scan_bf16_agg.hip -- scan_kernel instantiations: bf16 storage, kModeAgg.
#define SSM_IO BF16
#define SSM_MODE kModeAgg
#define SSM_RULE kRuleEuler
#include "scan_launch.inc"
