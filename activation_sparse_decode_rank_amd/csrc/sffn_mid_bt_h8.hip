// Small-batch middle kernel for fp16 weights and up to 8 tokens.
#include "sffn_mid_bt.h"

SFFN_MID_BT_ENTRY(true, 8, mid_bt_h8)
