// Host side of fa_softmax_fwd (include/fa.h): argument validation, choice of
// the kernel shape for the row length, and the launch on the caller's stream.
// No allocation, no synchronisation, no state.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "fa.h"
#include "softmax_table.h"

namespace {

bool pair_ok(int in_dtype, int out_dtype) {
    switch (in_dtype) {
        case FA_DTYPE_BF16: return out_dtype == FA_DTYPE_BF16 || out_dtype == FA_DTYPE_F32;
        case FA_DTYPE_F16: return out_dtype == FA_DTYPE_F16 || out_dtype == FA_DTYPE_F32;
        case FA_DTYPE_F32: return out_dtype == FA_DTYPE_F32;
        default: return false;
    }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" {

int fa_softmax_fwd(const void* x, void* y, float* lse, long long rows, int cols, fa_dtype_t in_dtype,
                   fa_dtype_t out_dtype, hipStream_t stream) {
    if (!x || !y) return FA_ERR_NULL;
    if (rows <= 0 || cols <= 0 || rows > INT32_MAX || rows * (long long)cols > (1LL << 40)) return FA_ERR_SHAPE;
    if (!pair_ok(in_dtype, out_dtype)) return FA_ERR_DTYPE;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(lse, 4)) return FA_ERR_ALIGN;
    const int in_bytes = in_dtype == FA_DTYPE_F32 ? 4 : 2;
    const int per_vec = 16 / in_bytes;
    const bool vec = cols % per_vec == 0;
    const long long nvec = cols / per_vec;
    // the smallest resident shape that holds the row, else a streamed form
    const fa::SoftmaxEntry* pick = nullptr;
    for (int i = 0; i < fa::kSoftmaxCount; ++i) {
        const fa::SoftmaxEntry& e = fa::kSoftmax[i];
        if (e.in_dtype != in_dtype || e.out_dtype != out_dtype) continue;
        if (e.kind == fa::kSmResident) {
            if (vec && !pick && nvec <= (long long)e.wpr * 64 * e.vpt) pick = &e;
        } else if (e.kind == fa::kSmResidentLds) {
            if (vec && !pick && nvec <= (long long)(e.vpt + e.vlds) * e.threads) pick = &e;
        } else if (!pick && e.kind == (vec ? fa::kSmStreamVec : fa::kSmStreamScalar)) {
            pick = &e;
        }
    }
    if (!pick) return FA_ERR_DTYPE;
    const long long rpb = pick->kind == fa::kSmResident ? pick->rpb : 1;  // one row per workgroup otherwise
    long long grid = (rows + rpb - 1) / rpb;
    // the register + LDS form walks rows with one workgroup per compute unit
    // of the 256
    if (pick->kind == fa::kSmResidentLds && grid > 256) grid = 256;
    fa::SoftmaxParams sp;
    sp.x = x;
    sp.y = y;
    sp.lse = lse;
    sp.rows = rows;
    sp.cols = cols;
    void* args[] = {&sp};
    const hipError_t err = hipLaunchKernel(pick->fn, dim3((unsigned)grid), dim3(pick->threads), args, 0,
                                           reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
