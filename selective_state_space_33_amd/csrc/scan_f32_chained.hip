// scan_f32_chained.hip -- scan_kernel instantiations: f32 storage, kModeChained.
#define SSM_IO F32
#define SSM_MODE kModeChained
#define SSM_RULE kRuleEuler
#include "scan_launch.inc"
