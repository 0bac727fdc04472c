/*
 * Drives every entry point of include/fa.h through its host-side paths, for
 * the AddressSanitizer / UndefinedBehaviorSanitizer build of the C ABI's host
 * code (linked against empty kernel tables, so no call reaches a launch).
 * Written in C11 to check that the public header is plain C.
 *
 * Every call carries either one invalid argument, which validation must
 * reject with the documented status, or valid arguments, which then stop at
 * the empty table lookup. Sizes near the overflow limits exercise the 64-bit
 * size arithmetic. Exit status 0 when every status is as expected.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa.h"

static int failures = 0;

#define EXPECT(expr, want)                                                                    \
    do {                                                                                      \
        long long got_ = (long long)(expr);                                                   \
        if (got_ != (long long)(want)) {                                                      \
            fprintf(stderr, "line %d: %s = %lld, expected %lld\n", __LINE__, #expr, got_,     \
                    (long long)(want));                                                       \
            ++failures;                                                                       \
        }                                                                                     \
    } while (0)

int main(void) {
    /* stand-in addresses, 16-byte aligned; never dereferenced */
    static _Alignas(16) unsigned char arena[256];
    void* P = arena;
    unsigned char* Pb = arena;
    float* L = (float*)arena;
    hipStream_t s = NULL;
    const fa_dtype_t BF = FA_DTYPE_BF16, F16 = FA_DTYPE_F16, F32 = FA_DTYPE_F32;

    /* fa_fwd / fa_fwd_ex: each invalid argument, then valid ones (no kernel) */
    EXPECT(fa_fwd(NULL, P, P, P, L, 1, 1, 8, 64, 0.1f, 0, NULL, BF, BF, s), FA_ERR_NULL);
    EXPECT(fa_fwd(P, P, P, P, NULL, 1, 1, 8, 64, 0.1f, 0, NULL, BF, BF, s), FA_ERR_NULL);
    EXPECT(fa_fwd(P, P, P, P, L, 0, 1, 8, 64, 0.1f, 0, NULL, BF, BF, s), FA_ERR_SHAPE);
    EXPECT(fa_fwd(P, P, P, P, L, 1, -3, 8, 64, 0.1f, 0, NULL, BF, BF, s), FA_ERR_SHAPE);
    EXPECT(fa_fwd(P, P, P, P, L, 1, 1, 8, 96, 0.1f, 0, NULL, BF, BF, s), FA_ERR_HEADDIM);
    EXPECT(fa_fwd(P, P, P, P, L, 1, 1, 8, 64, 0.1f, 0, NULL, BF, F16, s), FA_ERR_DTYPE);
    EXPECT(fa_fwd(P, P, P, P, L, 1, 1, 8, 64, 0.1f, 0, NULL, (fa_dtype_t)7, BF, s), FA_ERR_DTYPE);
    EXPECT(fa_fwd(P, P, P, P, L, 1, 1, 8, 64, -1.f, 0, NULL, BF, BF, s), FA_ERR_SCALE);
    EXPECT(fa_fwd(P, P, P, P, L, 1, 1, 8, 64, NAN, 0, NULL, BF, BF, s), FA_ERR_SCALE);
    EXPECT(fa_fwd(P, P, P, P, L, 1, 1, 8, 64, INFINITY, 0, NULL, BF, BF, s), FA_ERR_SCALE);
    EXPECT(fa_fwd(Pb + 8, P, P, P, L, 1, 1, 8, 64, 0.1f, 0, NULL, BF, BF, s), FA_ERR_ALIGN);
    EXPECT(fa_fwd(P, P, P, P, (float*)(Pb + 2), 1, 1, 8, 64, 0.1f, 0, NULL, BF, BF, s), FA_ERR_ALIGN);
    EXPECT(fa_fwd(P, P, P, P, L, 65536, 65536, 65536, 64, 0.1f, 0, NULL, BF, BF, s), FA_ERR_SHAPE);
    EXPECT(fa_fwd(P, P, P, P, L, 1, 1, 1 << 22, 128, 0.1f, 0, NULL, BF, BF, s), FA_ERR_SHAPE);
    EXPECT(fa_fwd(P, P, P, P, L, 2, 32, 8192, 128, 0.088f, 1, NULL, BF, BF, s), FA_ERR_TILE);
    EXPECT(fa_fwd(P, P, P, P, L, 8, 16, 4096, 64, 0.125f, 0, Pb, F16, F16, s), FA_ERR_TILE);
    EXPECT(fa_fwd(P, P, P, P, L, 1, 1, 256, 64, 0.125f, 0, NULL, F32, F32, s), FA_ERR_TILE);
    {
        fa_tile t = {96, 64};
        EXPECT(fa_fwd_ex(P, P, P, P, L, 1, 1, 8, 64, 0.1f, 0, NULL, BF, BF, s, &t), FA_ERR_TILE);
        t.block_r = -32;
        EXPECT(fa_fwd_ex(P, P, P, P, L, 1, 1, 8, 64, 0.1f, 0, NULL, BF, BF, s, &t), FA_ERR_TILE);
        EXPECT(fa_tile_supported(128, BF, BF, &t), FA_ERR_TILE);
        EXPECT(fa_tile_supported(128, BF, BF, NULL), FA_ERR_TILE);
        EXPECT(fa_default_tile(1, 8, 32768, 128, BF, BF, 1, 0, &t), FA_OK);
        EXPECT(t.block_r == 256 && t.block_c == 64, 1);
        EXPECT(fa_default_tile(1, 8, 8192, 128, BF, BF, 1, 0, &t), FA_OK);
        EXPECT(t.block_r == 128 && t.block_c == 32, 1);
        EXPECT(fa_default_tile(2, 32, 8192, 128, BF, BF, 1, 0, NULL), FA_ERR_NULL);
        EXPECT(fa_default_tile(1, 1, 0, 128, BF, BF, 1, 0, &t), FA_ERR_SHAPE);
        EXPECT(fa_default_tile(0, 1, 64, 128, BF, BF, 1, 0, &t), FA_ERR_SHAPE);
        EXPECT(fa_default_tile(1, -1, 64, 128, BF, BF, 1, 0, &t), FA_ERR_SHAPE);
        EXPECT(fa_default_tile(1, 1, 64, 32, BF, BF, 1, 0, &t), FA_ERR_HEADDIM);
        EXPECT(fa_default_tile(1, 1, 64, 64, F32, BF, 1, 0, &t), FA_ERR_DTYPE);
    }

    /* split-KV: workspace sizes, the split count over many shapes, the entry */
    EXPECT(fa_splitkv_workspace_bytes(2, 3, 100, 64, 4), 4LL * 2 * 3 * 100 * 65 * 4);
    EXPECT(fa_splitkv_workspace_bytes(65536, 65536, 65536, 64, 1), 0);
    EXPECT(fa_splitkv_workspace_bytes(1, 1, 8, 64, FA_MAX_SPLITS + 1), 0);
    for (int n = 1; n <= (1 << 20); n *= 3)
        for (int h = 1; h <= 64; h *= 4) {
            for (int causal = 0; causal < 2; ++causal) {
                const int a = fa_splitkv_num_splits(1, h, n, 128, BF, causal);
                const int b = fa_splitkv_num_splits(2, h, n, 64, F16, causal);
                const int c = fa_splitkv_num_splits(1, h, n, 128, F32, causal);
                EXPECT(a >= 1 && a <= 12 && b >= 1 && b <= 12 && c >= 1 && c <= 8, 1);
            }
        }
    EXPECT(fa_splitkv_num_splits(1, 1, 64, 80, BF, 0), FA_ERR_HEADDIM);
    EXPECT(fa_splitkv_num_splits(65536, 65536, 65536, 64, BF, 0) >= 1, 1);
    EXPECT(fa_splitkv_num_splits(65536, 65536, 65536, 64, BF, 1) >= 1, 1);
    EXPECT(fa_fwd_splitkv(P, P, P, P, L, 1, 1, 128, 128, 0.1f, 0, NULL, BF, BF, 0, P, 1 << 20, s), FA_ERR_SPLITS);
    EXPECT(fa_fwd_splitkv(P, P, P, P, L, 1, 1, 128, 128, 0.1f, 0, NULL, BF, BF, 2, NULL, 1 << 20, s),
           FA_ERR_WORKSPACE);
    EXPECT(fa_fwd_splitkv(P, P, P, P, L, 1, 1, 128, 128, 0.1f, 0, NULL, BF, BF, 2, P, 100, s), FA_ERR_WORKSPACE);
    EXPECT(fa_fwd_splitkv(P, P, P, P, L, 65536, 65536, 65536, 64, 0.1f, 0, NULL, BF, BF, 2, P, 1 << 20, s),
           FA_ERR_SHAPE);
    EXPECT(fa_fwd_splitkv(P, P, P, P, L, 1, 1, 128, 128, 0.1f, 1, NULL, BF, BF, 2, P, 1 << 20, s), FA_ERR_TILE);
    EXPECT(fa_fwd_splitkv_noalloc(P, P, P, P, L, 1, 64, 8192, 128, 0.1f, 0, NULL, BF, BF, 2, s), FA_ERR_SCRATCH);
    EXPECT(fa_fwd_splitkv_noalloc(P, P, P, P, L, 1, 1, 128, 128, 0.1f, 0, NULL, BF, BF, 65, s), FA_ERR_SPLITS);
    EXPECT(fa_fwd_splitkv_noalloc(P, P, P, P, L, 1, 1, 128, 128, 0.1f, 0, NULL, BF, F16, 2, s), FA_ERR_DTYPE);

    /* FP8 forward */
    EXPECT(fa_fwd_fp8(P, P, P, P, L, 1, 1, 128, 64, 0.1f, 1.f, 1.f, 1.f, 0, NULL, BF, 8, s), FA_ERR_HEADDIM);
    EXPECT(fa_fwd_fp8(P, P, P, P, L, 1, 1, 128, 128, 0.1f, 0.f, 1.f, 1.f, 0, NULL, BF, 8, s), FA_ERR_SCALE);
    EXPECT(fa_fwd_fp8(P, P, P, P, L, 1, 1, 128, 128, 0.1f, 1.f, 1.f, 1.f, 0, NULL, BF, 4, s), FA_ERR_OFFSET);
    EXPECT(fa_fwd_fp8(P, P, P, P, L, 2, 32, 8192, 128, 0.1f, 1.f, 1.f, 1.f, 1, NULL, BF, 8, s), FA_ERR_DTYPE);
    EXPECT(fa_fwd_fp8(P, P, P, P, L, 65536, 65536, 65536, 128, 0.1f, 1.f, 1.f, 1.f, 0, NULL, BF, 8, s), FA_ERR_SHAPE);

    /* backward */
    EXPECT(fa_bwd_workspace_bytes(2, 3, 100), 2LL * 3 * 4 * 64 * 4);
    EXPECT(fa_bwd_workspace_bytes(65536, 65536, 65536), 0);
    EXPECT(fa_bwd(P, P, P, P, P, L, P, P, P, 1, 1, 128, 128, 0.1f, 0, NULL, F32, F32, P, 1 << 20, s),
           FA_ERR_DTYPE);
    EXPECT(fa_bwd(P, P, P, P, P, L, P, P, P, 1, 1, 128, 128, 0.1f, 0, NULL, BF, BF, P, 4, s), FA_ERR_WORKSPACE);
    EXPECT(fa_bwd(P, P, P, P, P, L, P, P, P, 2, 4, 1000, 128, 0.1f, 1, Pb, BF, F32, P, 1 << 20, s), FA_ERR_TILE);

    /* row softmax */
    EXPECT(fa_softmax_fwd(P, P, L, 0, 64, BF, BF, s), FA_ERR_SHAPE);
    EXPECT(fa_softmax_fwd(P, P, L, (1LL << 31), 64, BF, BF, s), FA_ERR_SHAPE);
    EXPECT(fa_softmax_fwd(P, P, L, 1 << 30, 1 << 11, BF, BF, s), FA_ERR_SHAPE);
    EXPECT(fa_softmax_fwd(P, P, L, 4, 64, F32, BF, s), FA_ERR_DTYPE);
    EXPECT(fa_softmax_fwd(P, P, L, 4, 64, BF, BF, s), FA_ERR_DTYPE); /* no kernel registered */

    /* every status has a distinct name */
    for (int a = -12; a <= 0; ++a)
        for (int b = a + 1; b <= 0; ++b) EXPECT(strcmp(fa_strerror(a), fa_strerror(b)) != 0, 1);
    EXPECT(strcmp(fa_strerror(-99), "unknown status"), 0);

    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("capi host paths: ok\n");
    return 0;
}
