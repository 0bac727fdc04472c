// Registry of the FP8 attention-forward kernels (kern_fp8.hip).
#pragma once

#include "fa.h"

namespace fa {

struct Fp8Entry {
    int out_dtype, causal, mask, max_offset;
    const void* fn;
};

extern const Fp8Entry* const kFp8;
extern const int kFp8Count;

// Workgroup shape of the FP8 kernels: 4 waves of 32 queries.
constexpr int kFp8NW = 4;

}  // namespace fa
