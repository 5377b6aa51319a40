// scan_f32_ckpt.hip -- scan_kernel instantiations: f32 storage, kModeCkpt.
#define SSM_IO F32
#define SSM_MODE kModeCkpt
#define SSM_RULE kRuleEuler
#include "scan_launch.inc"
