// scan_bf16_n16.hip -- selective-scan kernels for bf16 io and up to 16 states.
#include "scan_kernel.h"

SFM_SCAN_INSTANCE(__bf16, bf16, 16)
