// scan_bf16_ckpt.hip -- scan_kernel instantiations: bf16 storage, kModeCkpt.
#define SSM_IO BF16
#define SSM_MODE kModeCkpt
#define SSM_RULE kRuleEuler
#include "scan_launch.inc"
