// Small-batch middle kernel for fp16 weights and up to 4 tokens.
#include "sffn_mid_bt.h"

SFFN_MID_BT_ENTRY(true, 4, mid_bt_h4)
