// Attention forward instantiations: head dim 128, bf16 inputs, bf16 or fp32 output.
#include "fa_table.h"

FA_DEFINE_LIST(d128_bf16, FA_TILES_D128, FA_SPLIT_D128, BF16, FA_DTYPE_BF16, F32, FA_DTYPE_F32)
