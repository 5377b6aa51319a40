// scan_bf16_ckptchain.hip -- scan_kernel instantiations: bf16 storage, kModeChainedCkpt.
#define SSM_IO BF16
#define SSM_MODE kModeChainedCkpt
#define SSM_RULE kRuleEuler
#include "scan_launch.inc"
