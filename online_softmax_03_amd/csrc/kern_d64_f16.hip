// Attention forward instantiations: head dim 64, f16 inputs, f16 or fp32 output.
#include "fa_table.h"

FA_DEFINE_LIST(d64_f16, FA_TILES_D64, FA_SPLIT_D64, F16, FA_DTYPE_F16, F32, FA_DTYPE_F32)
