// scan_f32_n16.hip -- selective-scan kernels for f32 io and up to 16 states.
#include "scan_kernel.h"

SFM_SCAN_INSTANCE(float, f32, 16)
