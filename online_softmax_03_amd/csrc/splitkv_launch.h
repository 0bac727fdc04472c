// Host side of the split-KV forward, shared by the entry points that take the
// partials' memory from the caller and from the library's own scratch.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace fa {

// FA_OK, or the status for the first invalid argument (the workspace aside).
int check_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                  float scale, int in_dtype, int out_dtype, int num_splits);

// Enqueues the split attention pass and the merge on `s`, with the partials in
// splitkv_bytes(B, H, N, d, num_splits) bytes at `ws` (16-byte aligned).
// Arguments must have passed check_splitkv.
int launch_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, const uint8_t* key_padding_mask, int in_dtype, int out_dtype,
                   int num_splits, void* ws, hipStream_t s);

}  // namespace fa
