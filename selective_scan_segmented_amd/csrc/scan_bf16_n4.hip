// scan_bf16_n4.hip -- selective-scan kernels for bf16 io and up to 4 states.
#include "scan_kernel.h"

SFM_SCAN_INSTANCE(__bf16, bf16, 4)
