// Registry of the row-softmax kernels (kern_softmax.hip); fa_api.hip picks
// one per call.
#pragma once

#include "fa.h"

namespace fa {

struct SoftmaxParams {
    const void* x;   // [rows][cols] of the input dtype
    void* y;         // [rows][cols] of the output dtype
    float* lse;      // [rows], or nullptr
    long long rows;
    int cols;
};

enum { kSmResident = 0, kSmStreamVec = 1, kSmStreamScalar = 2, kSmResidentLds = 3 };
constexpr int kSmStreamThreads = 256;

struct SoftmaxEntry {
    int in_dtype, out_dtype, kind;
    int wpr, rpb, vpt;  // resident shapes only
    int vlds;           // vectors per thread held in LDS (kSmResidentLds)
    int threads;
    const void* fn;
};

extern const SoftmaxEntry* const kSoftmax;
extern const int kSoftmaxCount;

}  // namespace fa
