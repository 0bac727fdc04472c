// Attention-backward instantiations for fp16 inputs: head dims 64 and 128,
// gradients in fp16 or fp32.
#include "attn_bwd_kernel.h"
#include "bwd_table.h"

#define FA_BWD_PAIR(D, TI, IN, TO, OUT, C, M)                                                               \
    fa::BwdEntry{fa::kBwdDq, D, IN, OUT, C, M,                                                              \
                 reinterpret_cast<const void*>(                                                             \
                     &fa::attn_bwd_dq_kernel<D, fa::kBwdBC, fa::kBwdNW, fa::TI, fa::TO, (C) != 0, (M) != 0>)}, \
        fa::BwdEntry{fa::kBwdDkdv, D, IN, OUT, C, M,                                                        \
                     reinterpret_cast<const void*>(&fa::attn_bwd_dkdv_kernel<D, fa::kBwdBQ, fa::kBwdNW, fa::TI, \
                                                                             fa::TO, (C) != 0, (M) != 0>)}
#define FA_BWD_FUSED(D, TI, IN, TO, OUT, C, M)                                                               \
    fa::BwdEntry{fa::kBwdFused, D, IN, OUT, C, M,                                                           \
                 reinterpret_cast<const void*>(&fa::attn_bwd_fused_kernel<D, fa::kBwdBC, fa::kBwdBQ, fa::kBwdNW,   \
                                                                          fa::TI, fa::TO, (C) != 0, (M) != 0>)}
#define FA_BWD_FUSED_FLAGS(D, TI, IN, TO, OUT)                                            \
    FA_BWD_FUSED(D, TI, IN, TO, OUT, 0, 0), FA_BWD_FUSED(D, TI, IN, TO, OUT, 0, 1),      \
        FA_BWD_FUSED(D, TI, IN, TO, OUT, 1, 0), FA_BWD_FUSED(D, TI, IN, TO, OUT, 1, 1)
#define FA_BWD_FLAGS(D, TI, IN, TO, OUT)                                                  \
    FA_BWD_PAIR(D, TI, IN, TO, OUT, 0, 0), FA_BWD_PAIR(D, TI, IN, TO, OUT, 0, 1),        \
        FA_BWD_PAIR(D, TI, IN, TO, OUT, 1, 0), FA_BWD_PAIR(D, TI, IN, TO, OUT, 1, 1)
#define FA_BWD_DTYPE(TI, IN)                                                                               \
    fa::BwdEntry{fa::kBwdPrep, 64, IN, -1, 0, 0, reinterpret_cast<const void*>(&fa::attn_bwd_prep_kernel<64, fa::TI>)}, \
        fa::BwdEntry{fa::kBwdPrep, 128, IN, -1, 0, 0,                                                      \
                     reinterpret_cast<const void*>(&fa::attn_bwd_prep_kernel<128, fa::TI>)},               \
        FA_BWD_FLAGS(64, TI, IN, TI, IN), FA_BWD_FLAGS(64, TI, IN, F32, FA_DTYPE_F32),                     \
        FA_BWD_FLAGS(128, TI, IN, TI, IN), FA_BWD_FLAGS(128, TI, IN, F32, FA_DTYPE_F32),                  \
        FA_BWD_FUSED_FLAGS(64, TI, IN, TI, IN), FA_BWD_FUSED_FLAGS(64, TI, IN, F32, FA_DTYPE_F32)

namespace fa {
static const BwdEntry kBwdEntries_f16[] = {FA_BWD_DTYPE(F16, FA_DTYPE_F16)};
extern const BwdList kBwdList_f16;
const BwdList kBwdList_f16 = {kBwdEntries_f16, (int)(sizeof(kBwdEntries_f16) / sizeof(kBwdEntries_f16[0]))};
}  // namespace fa
