// Split-KV merge kernels: head dims 64 and 128, every output dtype.
#include "fa_table.h"

namespace fa {
#define FA_MERGE(D, TO, OUT) MergeEntry{D, OUT, reinterpret_cast<const void*>(&attn_merge_kernel<D, TO>)}
static const MergeEntry kMergeEntries[] = {
    FA_MERGE(64, BF16, FA_DTYPE_BF16), FA_MERGE(64, F16, FA_DTYPE_F16), FA_MERGE(64, F32, FA_DTYPE_F32),
    FA_MERGE(128, BF16, FA_DTYPE_BF16), FA_MERGE(128, F16, FA_DTYPE_F16), FA_MERGE(128, F32, FA_DTYPE_F32),
};
extern const MergeEntry* const kMerge;
extern const int kMergeCount;
const MergeEntry* const kMerge = kMergeEntries;
const int kMergeCount = (int)(sizeof(kMergeEntries) / sizeof(kMergeEntries[0]));
}  // namespace fa
