// Row-softmax instantiations: every supported (input, output) dtype pair,
// the register-resident shapes and the two streamed forms.
#include "softmax_kernel.h"
#include "softmax_table.h"

namespace fa {

#define FA_SM_RES(TI, IN, TO, OUT, WPR, RPB, VPT)                 \
    SoftmaxEntry{IN, OUT, kSmResident, WPR, RPB, VPT, 0, WPR * RPB * 64, \
                 reinterpret_cast<const void*>(&softmax_resident_kernel<TI, TO, WPR, RPB, VPT>)}
#define FA_SM_RES_LDS(TI, IN, TO, OUT, NT, VPT, VLDS)                 \
    SoftmaxEntry{IN, OUT, kSmResidentLds, NT / 64, 1, VPT, VLDS, NT, \
                 reinterpret_cast<const void*>(&softmax_resident_lds_kernel<TI, TO, NT, VPT, VLDS>)}
#define FA_SM_STREAM(TI, IN, TO, OUT, VEC)                                               \
    SoftmaxEntry{IN, OUT, (VEC) ? kSmStreamVec : kSmStreamScalar, 0, 0, 0, 0, kSmStreamThreads, \
                 reinterpret_cast<const void*>(&softmax_stream_kernel<TI, TO, kSmStreamThreads, (VEC) != 0>)}
// Resident shapes, smallest first: (waves per row, rows per workgroup,
// vectors per thread); capacity = waves * 64 * vectors 16-byte vectors. Then
// the register + LDS shapes (threads, VPT vectors per thread in registers,
// VLDS in LDS): capacity (VPT + VLDS) * threads vectors. 1024 threads hold at
// most 128 registers each, 768 threads 168, so the largest shapes use 768
// threads with up to 13 LDS vectors (156 KB): 16384 and 20736 vectors for
// 16-bit inputs (each vector takes 8 registers as floats), 24576 and 33024
// for fp32 (4 registers each).
#define FA_SM_RES_ALL(TI, IN, TO, OUT)                                                        \
    FA_SM_RES(TI, IN, TO, OUT, 1, 4, 1), FA_SM_RES(TI, IN, TO, OUT, 1, 4, 2),               \
        FA_SM_RES(TI, IN, TO, OUT, 1, 4, 4), FA_SM_RES(TI, IN, TO, OUT, 2, 2, 4),           \
        FA_SM_RES(TI, IN, TO, OUT, 4, 1, 4), FA_SM_RES(TI, IN, TO, OUT, 8, 1, 4),           \
        FA_SM_RES(TI, IN, TO, OUT, 16, 1, 4), FA_SM_RES(TI, IN, TO, OUT, 16, 1, 8)
#define FA_SM_STREAMS(TI, IN, TO, OUT) FA_SM_STREAM(TI, IN, TO, OUT, 1), FA_SM_STREAM(TI, IN, TO, OUT, 0)
#define FA_SM_PAIR(TI, IN, TO, OUT)                                                                    \
    FA_SM_RES_ALL(TI, IN, TO, OUT), FA_SM_RES_LDS(TI, IN, TO, OUT, 1024, 8, 8), FA_SM_RES_LDS(TI, IN, TO, OUT, 768, 14, 13), \
        FA_SM_STREAMS(TI, IN, TO, OUT)
#define FA_SM_PAIR_F32(TI, IN, TO, OUT)                                                                  \
    FA_SM_RES_ALL(TI, IN, TO, OUT), FA_SM_RES_LDS(TI, IN, TO, OUT, 1024, 16, 8), FA_SM_RES_LDS(TI, IN, TO, OUT, 768, 31, 12), \
        FA_SM_STREAMS(TI, IN, TO, OUT)

static const SoftmaxEntry kSmEntries[] = {
    FA_SM_PAIR(BF16, FA_DTYPE_BF16, BF16, FA_DTYPE_BF16), FA_SM_PAIR(BF16, FA_DTYPE_BF16, F32, FA_DTYPE_F32),
    FA_SM_PAIR(F16, FA_DTYPE_F16, F16, FA_DTYPE_F16),     FA_SM_PAIR(F16, FA_DTYPE_F16, F32, FA_DTYPE_F32),
    FA_SM_PAIR_F32(F32, FA_DTYPE_F32, F32, FA_DTYPE_F32),
};
const SoftmaxEntry* const kSoftmax = kSmEntries;
const int kSoftmaxCount = (int)(sizeof(kSmEntries) / sizeof(kSmEntries[0]));

}  // namespace fa
