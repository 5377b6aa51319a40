// scan_bf16_full.hip -- scan_kernel instantiations: bf16 storage, kModeFull.
#define SSM_IO BF16
#define SSM_MODE kModeFull
#define SSM_RULE kRuleEuler
#include "scan_launch.inc"
