// Attention forward instantiations: fp32 inputs and output (fp32 MFMA), head
// dims 64 and 128, the default tile only (plain and split-KV).
#include "fa_table.h"

namespace fa {
#define FA_F32_ENTRY(D, C, M, S)                          \
    Entry{D, 64, 4, FA_DTYPE_F32, FA_DTYPE_F32, C, M, S, \
          reinterpret_cast<const void*>(&attn_fwd_f32_kernel<D, 64, 4, (C) != 0, (M) != 0, (S) != 0>)}
#define FA_F32_FLAGS(D, S) \
    FA_F32_ENTRY(D, 0, 0, S), FA_F32_ENTRY(D, 0, 1, S), FA_F32_ENTRY(D, 1, 0, S), FA_F32_ENTRY(D, 1, 1, S)
static const Entry kEntries_f32[] = {
    FA_F32_FLAGS(64, 0), FA_F32_FLAGS(64, 1), FA_F32_FLAGS(128, 0), FA_F32_FLAGS(128, 1),
};
extern const EntryList kList_f32;
const EntryList kList_f32 = {kEntries_f32, (int)(sizeof(kEntries_f32) / sizeof(kEntries_f32[0]))};
}  // namespace fa
