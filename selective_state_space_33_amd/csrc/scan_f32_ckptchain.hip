// scan_f32_ckptchain.hip -- scan_kernel instantiations: f32 storage, kModeChainedCkpt.
#define SSM_IO F32
#define SSM_MODE kModeChainedCkpt
#define SSM_RULE kRuleEuler
#include "scan_launch.inc"
