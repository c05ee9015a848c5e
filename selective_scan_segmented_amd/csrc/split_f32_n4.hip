// Lane-split selective-scan kernels for f32 io and 4 compiled states.
#include "scan_split.h"
SFM_SPLIT_INSTANCE(float, f32, 4, 2, 2)
