// Registry of compiled attention kernels: one Entry per (head dim, key tile,
// waves per workgroup, input/output dtype, causal, key mask) instantiation.
// Each kern_*.hip file instantiates one head dim and input dtype and exposes
// its entries; fa_api.hip searches them.
#pragma once

#include "attn_fwd_f32_kernel.h"
#include "attn_fwd_kernel.h"
#include "fa.h"

namespace fa {

struct Entry {
    int d, block_c, nwaves, in_dtype, out_dtype, causal, mask;
    const void* fn;
};

struct EntryList {
    const Entry* entries;
    int count;
};

}  // namespace fa

#define FA_ENTRY(D, BC, NW, TI, IN, TO, OUT, C, M) \
    fa::Entry{D, BC, NW, IN, OUT, C, M,            \
              reinterpret_cast<const void*>(&fa::attn_fwd_kernel<D, BC, NW, fa::TI, fa::TO, (C) != 0, (M) != 0>)}

#define FA_FLAGS(D, BC, NW, TI, IN, TO, OUT)                                                 \
    FA_ENTRY(D, BC, NW, TI, IN, TO, OUT, 0, 0), FA_ENTRY(D, BC, NW, TI, IN, TO, OUT, 0, 1), \
        FA_ENTRY(D, BC, NW, TI, IN, TO, OUT, 1, 0), FA_ENTRY(D, BC, NW, TI, IN, TO, OUT, 1, 1)

// Key-tile width B_c and waves per workgroup (B_r = 32 * waves) compiled per head dim.
#define FA_TILES_D128(TI, IN, TO, OUT) \
    FA_FLAGS(128, 64, 4, TI, IN, TO, OUT), FA_FLAGS(128, 32, 4, TI, IN, TO, OUT), FA_FLAGS(128, 64, 8, TI, IN, TO, OUT)

#define FA_TILES_D64(TI, IN, TO, OUT)                                                    \
    FA_FLAGS(64, 64, 4, TI, IN, TO, OUT), FA_FLAGS(64, 128, 4, TI, IN, TO, OUT),          \
        FA_FLAGS(64, 64, 8, TI, IN, TO, OUT), FA_FLAGS(64, 32, 4, TI, IN, TO, OUT)

// Defines fa::kList_<name>, the entries for both output dtypes of one input dtype.
#define FA_DEFINE_LIST(name, TILES, TI, IN, TO2, OUT2)                                   \
    namespace fa {                                                                      \
    static const Entry kEntries_##name[] = {TILES(TI, IN, TI, IN), TILES(TI, IN, TO2, OUT2)}; \
    extern const EntryList kList_##name;                                                \
    const EntryList kList_##name = {kEntries_##name,                                    \
                                    (int)(sizeof(kEntries_##name) / sizeof(kEntries_##name[0]))}; \
    }
