// Lane-split selective-scan kernels for bf16 io and 16 compiled states.
#include "scan_split.h"
SFM_SPLIT_INSTANCE(__bf16, bf16, 16, 2, 4)
