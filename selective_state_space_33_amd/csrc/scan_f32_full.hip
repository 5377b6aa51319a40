// scan_f32_full.hip -- scan_kernel instantiations: f32 storage, kModeFull.
#define SSM_IO F32
#define SSM_MODE kModeFull
#define SSM_RULE kRuleEuler
#include "scan_launch.inc"
