// Lane-split selective-scan kernels for bf16 io and 8 compiled states.
#include "scan_split.h"
SFM_SPLIT_INSTANCE(__bf16, bf16, 8, 2, 4)
