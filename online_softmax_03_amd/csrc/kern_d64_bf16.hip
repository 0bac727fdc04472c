// Attention forward instantiations: head dim 64, bf16 inputs, bf16 or fp32 output.
#include "fa_table.h"

FA_DEFINE_LIST(d64_bf16, FA_TILES_D64, FA_SPLIT_D64, BF16, FA_DTYPE_BF16, F32, FA_DTYPE_F32)
