// scan_f32_agg.hip -- scan_kernel instantiations: f32 storage, kModeAgg.
#define SSM_IO F32
#define SSM_MODE kModeAgg
#define SSM_RULE kRuleEuler
#include "scan_launch.inc"
