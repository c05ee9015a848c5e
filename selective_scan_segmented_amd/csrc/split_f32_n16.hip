// Lane-split selective-scan kernels for f32 io and 16 compiled states (lane groups of 2, 4 and 16).
#include "scan_split.h"
SFM_SPLIT_INSTANCE3(float, f32, 16, 2, 4, 16)
