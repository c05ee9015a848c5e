// Lane-split selective-scan kernels for bf16 io and 4 compiled states.
#include "scan_split.h"
SFM_SPLIT_INSTANCE(__bf16, bf16, 4, 2, 2)
