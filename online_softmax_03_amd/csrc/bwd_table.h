// Registry of the attention-backward kernels (kern_bwd_*.hip); bwd_api.hip
// picks them per call.
#pragma once

#include "fa.h"

namespace fa {

// Tile shapes of the backward: dQ walks key tiles of kBwdBC keys with
// kBwdNW waves (32 queries each); dK/dV walks query tiles of kBwdBQ queries
// with kBwdNW waves (32 keys each).
constexpr int kBwdNW = 4;
constexpr int kBwdBC = 32;
constexpr int kBwdBQ = 32;

// kBwdFused: dK/dV and dQ in one launch (attn_bwd_fused_kernel; d = 64).
enum { kBwdPrep = 0, kBwdDq = 1, kBwdDkdv = 2, kBwdFused = 3 };

struct BwdEntry {
    int kind, d, in_dtype, out_dtype, causal, mask;
    const void* fn;
};

struct BwdList {
    const BwdEntry* entries;
    int count;
};

}  // namespace fa
