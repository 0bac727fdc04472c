// Attention forward instantiations: fp32 inputs and output (fp32 MFMA), head
// dims 64 and 128, the default tile only.
#include "fa_table.h"

namespace fa {
static const Entry kEntries_f32[] = {
    FA_FLAGS(64, 64, 4, F32, FA_DTYPE_F32, F32, FA_DTYPE_F32),
    FA_FLAGS(128, 64, 4, F32, FA_DTYPE_F32, F32, FA_DTYPE_F32),
};
extern const EntryList kList_f32;
const EntryList kList_f32 = {kEntries_f32, (int)(sizeof(kEntries_f32) / sizeof(kEntries_f32[0]))};
}  // namespace fa
