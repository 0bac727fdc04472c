// Registry of compiled attention kernels: one Entry per (head dim, key tile,
// waves per workgroup, input/output dtype, causal, key mask, split-KV)
// instantiation.
// Each kern_*.hip file instantiates one head dim and input dtype and exposes
// its entries; fa_api.hip searches them.
#pragma once

#include "attn_fwd_f32_kernel.h"
#include "attn_fwd_kernel.h"
#include "attn_merge.h"
#include "fa.h"

namespace fa {

struct Entry {
    int d, block_c, nwaves, in_dtype, out_dtype, causal, mask, split;
    const void* fn;
};

// Merge kernels of the split-KV path, one per (d, output dtype).
struct MergeEntry {
    int d, out_dtype;
    const void* fn;
};

struct EntryList {
    const Entry* entries;
    int count;
};

}  // namespace fa

#define FA_ENTRY(D, BC, NW, TI, IN, TO, OUT, C, M, S)                                                    \
    fa::Entry{D, BC, NW, IN, OUT, C, M, S,                                                              \
              reinterpret_cast<const void*>(                                                        \
                  &fa::attn_fwd_kernel<D, BC, NW, fa::TI, fa::TO, (C) != 0, (M) != 0, (S) != 0>)}

#define FA_FLAGS_S(D, BC, NW, TI, IN, TO, OUT, S)                                                     \
    FA_ENTRY(D, BC, NW, TI, IN, TO, OUT, 0, 0, S), FA_ENTRY(D, BC, NW, TI, IN, TO, OUT, 0, 1, S),     \
        FA_ENTRY(D, BC, NW, TI, IN, TO, OUT, 1, 0, S), FA_ENTRY(D, BC, NW, TI, IN, TO, OUT, 1, 1, S)
#define FA_FLAGS(D, BC, NW, TI, IN, TO, OUT) FA_FLAGS_S(D, BC, NW, TI, IN, TO, OUT, 0)

// Key-tile width B_c and waves per workgroup (B_r = 32 * waves) compiled per
// head dim.
#define FA_TILES_D128(TI, IN, TO, OUT) \
    FA_FLAGS(128, 64, 4, TI, IN, TO, OUT), FA_FLAGS(128, 32, 4, TI, IN, TO, OUT), FA_FLAGS(128, 64, 8, TI, IN, TO, OUT)

#define FA_TILES_D64(TI, IN, TO, OUT)                                                    \
    FA_FLAGS(64, 64, 4, TI, IN, TO, OUT), FA_FLAGS(64, 128, 4, TI, IN, TO, OUT),          \
        FA_FLAGS(64, 64, 8, TI, IN, TO, OUT), FA_FLAGS(64, 32, 4, TI, IN, TO, OUT)

// The split-KV form (fp32 partials to a workspace, so one per input dtype) of
// the default tile only.
#define FA_SPLIT_D128(TI, IN) FA_FLAGS_S(128, 32, 4, TI, IN, TI, IN, 1)
#define FA_SPLIT_D64(TI, IN) FA_FLAGS_S(64, 64, 8, TI, IN, TI, IN, 1)

#define FA_DEFINE_LIST(name, TILES, SPLITS, TI, IN, TO2, OUT2)                           \
    namespace fa {                                                                      \
    static const Entry kEntries_##name[] = {TILES(TI, IN, TI, IN), TILES(TI, IN, TO2, OUT2), \
                                            SPLITS(TI, IN)};                            \
    extern const EntryList kList_##name;                                                \
    const EntryList kList_##name = {kEntries_##name,                                    \
                                    (int)(sizeof(kEntries_##name) / sizeof(kEntries_##name[0]))}; \
    }
