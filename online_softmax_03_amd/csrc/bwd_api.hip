// Host side of fa_bwd (include/fa.h): argument validation, kernel choice and
// the launches on the caller's stream: prep, then dK/dV and dQ (one fused
// launch at d = 64, two at d = 128). No
// allocation, no synchronisation, no state.
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "attn_bwd_kernel.h"
#include "bwd_table.h"
#include "fa.h"

namespace fa {
extern const BwdList kBwdList_bf16, kBwdList_f16;
}

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

const fa::BwdEntry* find(int kind, int d, int in_dtype, int out_dtype, int causal, int mask) {
    const fa::BwdList* lists[] = {&fa::kBwdList_bf16, &fa::kBwdList_f16};
    for (const fa::BwdList* l : lists)
        for (int i = 0; i < l->count; ++i) {
            const fa::BwdEntry& e = l->entries[i];
            if (e.kind != kind || e.d != d || e.in_dtype != in_dtype) continue;
            if (kind == fa::kBwdPrep) return &e;
            if (e.out_dtype == out_dtype && e.causal == (causal != 0) && e.mask == (mask != 0)) return &e;
        }
    return nullptr;
}

// 32-query groups per head, padded to a multiple of 64 queries.
long long groups(int N) { return 2 * (((long long)N + 63) / 64); }

}  // namespace

extern "C" {

size_t fa_bwd_workspace_bytes(int B, int H, int N) {
    if (B <= 0 || H <= 0 || N <= 0) return 0;
    const long long rows = (long long)B * H * N;
    if (rows > (1LL << 40)) return 0;
    return (size_t)B * (size_t)H * (size_t)groups(N) * 64 * sizeof(float);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
           const uint8_t* key_padding_mask, fa_dtype_t in_dtype, fa_dtype_t grad_dtype, void* workspace,
           size_t workspace_bytes, hipStream_t stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (!((in_dtype == FA_DTYPE_BF16 || in_dtype == FA_DTYPE_F16) &&
          (grad_dtype == in_dtype || grad_dtype == FA_DTYPE_F32)))
        return FA_ERR_DTYPE;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    const size_t need = fa_bwd_workspace_bytes(B, H, N);
    if (need == 0) return FA_ERR_SHAPE;
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return FA_ERR_WORKSPACE;
    const fa::BwdEntry* prep = find(fa::kBwdPrep, d, in_dtype, grad_dtype, causal, key_padding_mask != nullptr);
    const fa::BwdEntry* edq = find(fa::kBwdDq, d, in_dtype, grad_dtype, causal, key_padding_mask != nullptr);
    const fa::BwdEntry* ekv = find(fa::kBwdDkdv, d, in_dtype, grad_dtype, causal, key_padding_mask != nullptr);
    if (!prep || !edq || !ekv) return FA_ERR_TILE;
    // d = 64: dK/dV and dQ in one launch (attn_bwd_fused_kernel)
    const fa::BwdEntry* efu =
        d == 64 ? find(fa::kBwdFused, d, in_dtype, grad_dtype, causal, key_padding_mask != nullptr) : nullptr;

    const long long bh = (long long)B * H;
    const long long n_g = groups(N);
    const long long n_qtiles = ((long long)N + fa::kBwdNW * 32 - 1) / (fa::kBwdNW * 32);
    const long long n_ktiles = n_qtiles;  // key tiles have the same height
    const long long prep_rows_per_block = 256 / (d / 8);
    const long long prep_grid = (bh * n_g * 32 + prep_rows_per_block - 1) / prep_rows_per_block;
    const long long grid = bh * n_qtiles;
    if ((long long)N * d * 4 > INT32_MAX || 2 * grid > INT32_MAX || prep_grid > INT32_MAX) return FA_ERR_SHAPE;

    fa::BwdParams prm;
    prm.q = q;
    prm.k = k;
    prm.v = v;
    prm.o = o;
    prm.dout = dout;
    prm.lse = lse;
    prm.stats = static_cast<float*>(workspace);
    prm.dq = dq;
    prm.dk = dk;
    prm.dv = dv;
    prm.mask = key_padding_mask;
    prm.B = B;
    prm.H = H;
    prm.N = N;
    prm.n_g = (int)n_g;
    prm.n_qtiles = (int)n_qtiles;
    prm.n_ktiles = (int)n_ktiles;
    prm.xcd_remap = fa::xcd_mode_for(B * H, grid);
    prm.head_group = fa::head_group_for(B * H, causal);
    // Groups of four heads when every XCD holds a multiple of four (B*H a
    // multiple of 32), as for the forward: causal N = 8192, 64 heads, three
    // alternating bench runs each, 860 against 850 TFLOP/s with pairs.
    if (causal && (long long)B * H % 32 == 0) prm.head_group = 4;
    prm.n_dkdv_blocks = (int)grid;
    prm.c = (float)((double)scale * 1.4426950408889634074);
    prm.scale = scale;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    void* args[] = {&prm};
    if (hipLaunchKernel(prep->fn, dim3((unsigned)prep_grid), dim3(256), args, 0, s) != hipSuccess)
        return FA_ERR_LAUNCH;
    if (efu) {
        if (hipLaunchKernel(efu->fn, dim3((unsigned)(2 * grid)), dim3(fa::kBwdNW * 64), args, 0, s) != hipSuccess)
            return FA_ERR_LAUNCH;
        return FA_OK;
    }
    if (hipLaunchKernel(ekv->fn, dim3((unsigned)grid), dim3(fa::kBwdNW * 64), args, 0, s) != hipSuccess)
        return FA_ERR_LAUNCH;
    if (hipLaunchKernel(edq->fn, dim3((unsigned)grid), dim3(fa::kBwdNW * 64), args, 0, s) != hipSuccess)
        return FA_ERR_LAUNCH;
    return FA_OK;
}

}  // extern "C"
