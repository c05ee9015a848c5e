// Lane-split selective-scan kernels for f32 io and 16 compiled states.
#include "scan_split.h"
SFM_SPLIT_INSTANCE(float, f32, 16, 2, 4)
