// Host side of fa_fwd_fp8 (include/fa.h): validation, kernel choice and the
// launch on the caller's stream. No allocation, no synchronisation, no state.
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "attn_fwd_fp8_kernel.h"
#include "fa.h"
#include "fp8_table.h"

namespace {
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool pos_finite(float x) { return x > 0.f && isfinite(x); }
}  // namespace

extern "C" {

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, float descale_q, float descale_k, float descale_v, int causal,
               const uint8_t* key_padding_mask, fa_dtype_t out_dtype, int max_offset, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_SHAPE;
    if (d != 128) return FA_ERR_HEADDIM;
    if (out_dtype != FA_DTYPE_BF16 && out_dtype != FA_DTYPE_F16 && out_dtype != FA_DTYPE_F32) return FA_ERR_DTYPE;
    if (!pos_finite(scale) || !pos_finite(descale_q) || !pos_finite(descale_k) || !pos_finite(descale_v))
        return FA_ERR_SCALE;
    if (max_offset != 0 && max_offset != 8) return FA_ERR_OFFSET;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    const long long rows = (long long)B * H * N;
    const long long n_qtiles = ((long long)N + fa::kFp8NW * 32 - 1) / (fa::kFp8NW * 32);
    const long long grid = (long long)B * H * n_qtiles;
    if (rows > (1LL << 40) || (long long)N * d * 4 > INT32_MAX || grid > INT32_MAX) return FA_ERR_SHAPE;
    const fa::Fp8Entry* e = nullptr;
    for (int i = 0; i < fa::kFp8Count; ++i) {
        const fa::Fp8Entry& x = fa::kFp8[i];
        if (x.out_dtype == out_dtype && x.causal == (causal != 0) && x.mask == (key_padding_mask != nullptr) &&
            x.max_offset == max_offset)
            e = &x;
    }
    if (!e) return FA_ERR_DTYPE;
    fa::ParamsFp8 prm;
    prm.q = q;
    prm.k = k;
    prm.v = v;
    prm.o = o;
    prm.lse = lse;
    prm.mask = key_padding_mask;
    prm.B = B;
    prm.H = H;
    prm.N = N;
    prm.n_qtiles = (int)n_qtiles;
    prm.xcd_remap = fa::xcd_mode_for(B * H, grid);
    prm.head_group = fa::head_group_for(B * H, causal);
    // Groups of four heads when every XCD holds a multiple of four (B*H a
    // multiple of 32), as for the 16-bit forward: same process, causal
    // N = 8192, 64 heads, G = 4 0.5591-0.5621 ms against G = 2 0.5701-0.5804.
    if (causal && (long long)B * H % 32 == 0) prm.head_group = 4;
    prm.c = (float)((double)scale * descale_q * descale_k * 1.4426950408889634074);
    prm.descale_v = descale_v;
    void* args[] = {&prm};
    const hipError_t err = hipLaunchKernel(e->fn, dim3((unsigned)grid), dim3(fa::kFp8NW * 64), args, 0,
                                           reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
