// FP8 (E4M3) attention-forward instantiations: head dim 128, outputs bf16,
// fp16 or fp32, Max_offset 8 (the FP8 setting) or 0 (for comparison).
#include "attn_fwd_fp8_kernel.h"
#include "fp8_table.h"

#define FA_FP8_ENTRY(TO, OUT, C, M, OFF) \
    fa::Fp8Entry{OUT, C, M, OFF, reinterpret_cast<const void*>(&fa::attn_fwd_fp8_kernel<128, 4, fa::TO, (C) != 0, (M) != 0, OFF>)}
#define FA_FP8_FLAGS(TO, OUT, OFF)                                                           \
    FA_FP8_ENTRY(TO, OUT, 0, 0, OFF), FA_FP8_ENTRY(TO, OUT, 0, 1, OFF), FA_FP8_ENTRY(TO, OUT, 1, 0, OFF), \
        FA_FP8_ENTRY(TO, OUT, 1, 1, OFF)
#define FA_FP8_OUT(TO, OUT) FA_FP8_FLAGS(TO, OUT, 8), FA_FP8_FLAGS(TO, OUT, 0)

namespace fa {
static const Fp8Entry kFp8Entries[] = {
    FA_FP8_OUT(BF16, FA_DTYPE_BF16), FA_FP8_OUT(F16, FA_DTYPE_F16), FA_FP8_OUT(F32, FA_DTYPE_F32),
};
const Fp8Entry* const kFp8 = kFp8Entries;
const int kFp8Count = (int)(sizeof(kFp8Entries) / sizeof(kFp8Entries[0]));
}  // namespace fa
