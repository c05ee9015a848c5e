// Lane-split selective-scan kernels for bf16 io and 16 compiled states (lane groups of 2, 4 and 16).
#include "scan_split.h"
SFM_SPLIT_INSTANCE3(__bf16, bf16, 16, 2, 4, 16)
