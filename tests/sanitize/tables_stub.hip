// Empty kernel tables for the sanitizer build of the C ABI's host code: with
// no kernel registered, every call that passes argument validation stops at
// the table lookup, so the driver exercises validation and size arithmetic
// without a GPU and without a kernel launch.
#include "attn_merge.h"
#include "bwd_table.h"
#include "fa_table.h"
#include "fp8_table.h"
#include "softmax_table.h"

namespace fa {
extern const EntryList kList_d128_bf16, kList_d128_f16, kList_d64_bf16, kList_d64_f16, kList_f32;
const EntryList kList_d128_bf16 = {nullptr, 0};
const EntryList kList_d128_f16 = {nullptr, 0};
const EntryList kList_d64_bf16 = {nullptr, 0};
const EntryList kList_d64_f16 = {nullptr, 0};
const EntryList kList_f32 = {nullptr, 0};
extern const MergeEntry* const kMerge;
extern const int kMergeCount;
const MergeEntry* const kMerge = nullptr;
const int kMergeCount = 0;
extern const BwdList kBwdList_bf16, kBwdList_f16;
const BwdList kBwdList_bf16 = {nullptr, 0};
const BwdList kBwdList_f16 = {nullptr, 0};
const Fp8Entry* const kFp8 = nullptr;
const int kFp8Count = 0;
const SoftmaxEntry* const kSoftmax = nullptr;
const int kSoftmaxCount = 0;
}  // namespace fa
