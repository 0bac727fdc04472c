// fa_fwd_splitkv_noalloc (include/fa.h): the split-KV forward for callers that
// cannot allocate device memory. The split partials go to a fixed array that
// the library's code object holds on every device; the entry point looks up
// its device address once per device and otherwise calls no allocator.
#include <stdint.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "fa.h"
#include "splitkv_launch.h"

namespace {

// The fixed scratch: float32 partial outputs, then their LSEs, as in the
// caller's workspace of fa_fwd_splitkv. In host code this name is only a
// stand-in for the device symbol, never an address the device can use.
__device__ __align__(256) static char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch`, per device; null until looked up

// The address of `scratch` on the calling thread's current device.
int scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FA_ERR_LAUNCH;
        g_ptr[dev] = ptr;
    }
    *out = g_ptr[dev];
    return FA_OK;
}

// Sizes as fa_splitkv_workspace_bytes computes them (0 when out of range).
size_t partial_bytes(int B, int H, int N, int d, int S) {
    const long long rows = (long long)B * H * N;
    if (rows > (1LL << 40)) return 0;
    return (size_t)S * (size_t)rows * (size_t)(d + 1) * sizeof(float);
}

}  // namespace

extern "C" {

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                           int N, int d, float scale, int causal, const uint8_t* key_padding_mask,
                           fa_dtype_t in_dtype, fa_dtype_t out_dtype, int num_splits, hipStream_t stream) {
    const int st = fa::check_splitkv(q, k, v, o, lse, B, H, N, d, scale, in_dtype, out_dtype, num_splits);
    if (st != FA_OK) return st;
    if (partial_bytes(B, H, N, d, num_splits) > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    void* ws = nullptr;
    const int sst = scratch_on_current_device(&ws);
    if (sst != FA_OK) return sst;
    return fa::launch_splitkv(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask, in_dtype, out_dtype,
                              num_splits, ws, stream);
}

}  // extern "C"
