// Small-batch middle kernel for fp32 weights and up to 4 tokens.
#include "sffn_mid_bt.h"

SFFN_MID_BT_ENTRY(false, 4, mid_bt_f4)
