// Attention forward instantiations: head dim 128, f16 inputs, f16 or fp32 output.
#include "fa_table.h"

FA_DEFINE_LIST(d128_f16, FA_TILES_D128, FA_SPLIT_D128, F16, FA_DTYPE_F16, F32, FA_DTYPE_F32)
