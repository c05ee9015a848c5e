// scan_f32_n8.hip -- selective-scan kernels for f32 io and up to 8 states.
#include "scan_kernel.h"

SFM_SCAN_INSTANCE(float, f32, 8)
