// Host side of the C ABI declared in include/fa.h: argument validation, tile
// selection, and the kernel launch on the caller's stream. No allocation, no
// synchronisation, no state.
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "fa.h"
#include "fa_table.h"
#include "splitkv_launch.h"

namespace fa {
extern const EntryList kList_d128_bf16, kList_d128_f16, kList_d64_bf16, kList_d64_f16, kList_f32;
extern const MergeEntry* const kMerge;
extern const int kMergeCount;
}

namespace {

using fa::Entry;

const fa::EntryList* const kLists[] = {&fa::kList_d128_bf16, &fa::kList_d128_f16, &fa::kList_d64_bf16,
                                       &fa::kList_d64_f16, &fa::kList_f32};

bool dtype_pair_ok(int in_dtype, int out_dtype) {
    switch (in_dtype) {
        case FA_DTYPE_BF16: return out_dtype == FA_DTYPE_BF16 || out_dtype == FA_DTYPE_F32;
        case FA_DTYPE_F16: return out_dtype == FA_DTYPE_F16 || out_dtype == FA_DTYPE_F32;
        case FA_DTYPE_F32: return out_dtype == FA_DTYPE_F32;
        default: return false;
    }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Base tiles from the tile sweep on MI355X: for 16-bit inputs, d = 128 with
// 128 query rows and 32-key tiles (three waves per SIMD; the split-KV forms
// and the key-masked launches of short sequences use it) and d = 64 with 256
// query rows and 64-key tiles. fp32 inputs have one tile shape, 128 x 64.
fa_tile default_tile(int d, int in_dtype) {
    if (in_dtype == FA_DTYPE_F32) return fa_tile{128, 64};
    return d == 128 ? fa_tile{128, 32} : fa_tile{256, 64};
}

// The tile fa_fwd takes when the caller names none. For 16-bit d = 128,
// 256 x 64 (eight waves sharing every 64-key tile: half the LDS fills, waits
// and barriers per MFMA of 128 x 32, at two waves per SIMD) is ahead where
// each workgroup's key loop is long and the grid of 256-row tiles, G, is
// between about one and four workgroups per CU. Same-process A/B on three
// MI355X cards: causal N = 8192 at G = 384 +17%, G = 512 +2.5-3.4%, N = 16384 at
// G = 512 +2.5-3.5%, N = 32768 at G = 1024 +0.7-3.5%; non-causal N = 8192 at
// G = 256 +10-11%, 512 +7%, 1024 +2-5%, N = 4096 at G = 1024 +2-3%. Behind
// or tied with short loops (causal N <= 6144: -0.1 to -2.4%, non-causal
// N = 2048: -0.7%), with G <= 256 under a causal mask (-4.9 to -5.9%) and
// with larger causal grids (N = 8192 at G = 2048: -0.6 to +1.8%, N = 16384
// at G = 4096: -2.4%).
fa_tile auto_tile(int B, int H, int N, int d, int in_dtype, int causal) {
    const fa_tile t = default_tile(d, in_dtype);
    if (in_dtype == FA_DTYPE_F32 || d != 128) return t;
    const long long G = (long long)B * H * ((N + 255) / 256);
    const bool wide = causal ? (N >= 8192 && G >= 384 && G <= 1024) : (N >= 4096 && G >= 256 && G <= 1024);
    return wide ? fa_tile{256, 64} : t;
}

// The split-KV kernels write fp32 partials whatever the final output dtype,
// so for them the output dtype is not part of the match.
const Entry* find(int d, const fa_tile& t, int in_dtype, int out_dtype, int causal, int mask,
                  int split = 0) {
    if (t.block_r <= 0 || t.block_r % 32 != 0) return nullptr;
    const int nw = t.block_r / 32;
    for (const fa::EntryList* list : kLists) {
        for (int i = 0; i < list->count; ++i) {
            const Entry& e = list->entries[i];
            if (e.d == d && e.block_c == t.block_c && e.nwaves == nw && e.in_dtype == in_dtype &&
                (split || e.out_dtype == out_dtype) && e.causal == (causal != 0) && e.mask == (mask != 0) &&
                e.split == split)
                return &e;
        }
    }
    return nullptr;
}

const fa::MergeEntry* find_merge(int d, int out_dtype) {
    for (int i = 0; i < fa::kMergeCount; ++i)
        if (fa::kMerge[i].d == d && fa::kMerge[i].out_dtype == out_dtype) return &fa::kMerge[i];
    return nullptr;
}

// Workgroups of the default-tile split-KV kernel that one compute unit holds
// at once (its register use): 3 for the 16-bit d = 128 tile (4 waves of at
// most 168 VGPRs, a bound its split and key-masked forms carry), 2 for the
// 16-bit d = 64 tile (8 waves of at most 128) and for the fp32 d = 64 tile
// (4 waves of at most 256), 1 for the fp32 d = 128 tile (4 waves of 256
// VGPRs plus AGPRs).
int resident_wgs_per_cu(int d, int in_dtype) {
    if (in_dtype == FA_DTYPE_F32) return d == 128 ? 1 : 2;
    return d == 128 ? 3 : 2;
}

// Workspace of the split-KV path: fp32 partial outputs [S][B*H*N][d], then
// their LSEs [S][B*H*N]. 0 if the sizes are out of range.
size_t splitkv_bytes(int B, int H, int N, int d, int S) {
    if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128) || S < 1 || S > FA_MAX_SPLITS) return 0;
    const long long rows = (long long)B * H * N;
    if (rows > (1LL << 40)) return 0;
    return (size_t)S * (size_t)rows * (size_t)(d + 1) * sizeof(float);
}

// The parts of a split-KV launch with the default tile. Under a causal mask,
// for 16-bit inputs, when the unsplit launch has no more query tiles than
// there are CUs (B*H*ceil(N/block_r) <= 256), query tile qt gets parts in
// proportion to its causal extent: at most u * block_r / block_c key tiles
// each, num_splits (at most) for the last tile (parts_of, work_item.h). Every
// query tile otherwise gets num_splits parts. Same-card comparisons on causal
// d = 128, N = 8192 (TFLOP/s, equal parts against proportional parts, at the
// best part count of each): 1 head 369 / 418, 2 heads 454 / 584, 4 heads 630
// / 691; 8 heads 866 / 786 (512 query tiles: equal parts, 1024 workgroups of
// all lengths, fill the slots better than 768 equal ones) and 8 heads at
// N = 4096 (256 query tiles) 576 / 568.
struct SplitPlan {
    int u;             // 0: num_splits equal parts for every query tile
    int s_last;        // parts of the longest query tile (<= num_splits)
    long long parts;   // workgroups per head
};

SplitPlan split_plan(int B, int H, int N, int d, int in_dtype, int causal, int num_splits) {
    const fa_tile t = default_tile(d, in_dtype);
    const long long n_qtiles = ((long long)N + t.block_r - 1) / t.block_r;
    SplitPlan sp{0, num_splits, n_qtiles * num_splits};
    if (causal && in_dtype != FA_DTYPE_F32 && (long long)B * H * n_qtiles <= 256) {
        const int r = t.block_r / t.block_c;
        const int n_k = (N + t.block_c - 1) / t.block_c;
        sp.u = fa::split_unit(n_k, r, num_splits);
        sp.s_last = (n_k + sp.u * r - 1) / (sp.u * r);
        sp.parts = fa::parts_per_head((int)n_qtiles, sp.u, sp.s_last);
    }
    return sp;
}

// Shared argument checks of fa_fwd_ex and fa_fwd_splitkv.
int check_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                 int d, float scale, int in_dtype, int out_dtype) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (!dtype_pair_ok(in_dtype, out_dtype)) return FA_ERR_DTYPE;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    return FA_OK;
}

void fill_params(fa::Params& prm, const void* q, const void* k, const void* v, void* o, float* lse,
                 const uint8_t* mask, int B, int H, int N, float scale, int causal, long long n_qtiles,
                 long long grid) {
    prm.q = q;
    prm.k = k;
    prm.v = v;
    prm.o = o;
    prm.lse = lse;
    prm.mask = mask;
    prm.B = B;
    prm.H = H;
    prm.N = N;
    prm.n_qtiles = (int)n_qtiles;
    prm.xcd_remap = fa::xcd_mode_for(B * H, grid);
    prm.head_group = fa::head_group_for(B * H, causal);
    prm.fair = 0;
    prm.c = (float)((double)scale * 1.4426950408889634074);  // scale * log2(e)
    prm.n_splits = 1;
    prm.split_u = 0;
    prm.split_parts = 0;
    prm.ws_o = nullptr;
    prm.ws_lse = nullptr;
}

// The caller's tile: NULL or {0, 0} is the library's choice for the shape;
// a zero in one field takes that field from the base tile.
fa_tile resolve(int B, int H, int N, int d, int in_dtype, int causal, const fa_tile* tile) {
    if (!tile || (tile->block_r == 0 && tile->block_c == 0)) return auto_tile(B, H, N, d, in_dtype, causal);
    fa_tile t = default_tile(d, in_dtype);
    if (tile->block_r != 0) t.block_r = tile->block_r;
    if (tile->block_c != 0) t.block_c = tile->block_c;
    return t;
}


}  // namespace

namespace fa {

// Argument checks of the split-KV entry points, everything but the
// workspace (declared in splitkv_launch.h).
int check_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                  float scale, int in_dtype, int out_dtype, int num_splits) {
    const int st = check_common(q, k, v, o, lse, B, H, N, d, scale, in_dtype, out_dtype);
    if (st != FA_OK) return st;
    if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
    if (splitkv_bytes(B, H, N, d, num_splits) == 0) return FA_ERR_SHAPE;
    const fa_tile t = default_tile(d, in_dtype);
    const long long rows = (long long)B * H * N;
    const long long n_qtiles = ((long long)N + t.block_r - 1) / t.block_r;
    const long long grid = (long long)B * H * n_qtiles * num_splits;
    const long long rows_per_block = 256 / (d / 4);
    const long long merge_grid = (rows + rows_per_block - 1) / rows_per_block;
    if ((long long)N * d * 4 > INT32_MAX || grid > INT32_MAX || merge_grid > INT32_MAX) return FA_ERR_SHAPE;
    return FA_OK;
}

// The split attention pass and the merge, on a workspace of
// splitkv_bytes(B, H, N, d, num_splits) bytes at `ws` (arguments already
// checked by check_splitkv).
int launch_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, const uint8_t* key_padding_mask, int in_dtype, int out_dtype,
                   int num_splits, void* ws, hipStream_t s) {
    const fa_tile t = default_tile(d, in_dtype);
    const Entry* e = find(d, t, in_dtype, out_dtype, causal, key_padding_mask != nullptr, 1);
    const fa::MergeEntry* me = find_merge(d, out_dtype);
    if (!e || !me) return FA_ERR_TILE;
    const long long rows = (long long)B * H * N;
    const long long n_qtiles = ((long long)N + t.block_r - 1) / t.block_r;
    const SplitPlan sp = split_plan(B, H, N, d, in_dtype, causal, num_splits);
    const int u = sp.u, s_last = sp.s_last;
    const long long parts = sp.parts;
    const long long grid = (long long)B * H * parts;
    const long long rows_per_block = 256 / (d / 4);
    const long long merge_grid = (rows + rows_per_block - 1) / rows_per_block;

    float* ws_o = static_cast<float*>(ws);
    float* ws_lse = ws_o + (size_t)num_splits * (size_t)rows * (size_t)d;
    fa::Params prm;
    fill_params(prm, q, k, v, o, lse, key_padding_mask, B, H, N, scale, causal, n_qtiles, grid);
    prm.n_splits = s_last;
    prm.split_u = u;
    prm.split_parts = parts;
    prm.ws_o = ws_o;
    prm.ws_lse = ws_lse;
    void* args[] = {&prm};
    if (hipLaunchKernel(e->fn, dim3((unsigned)grid), dim3(e->nwaves * 64), args, 0, s) != hipSuccess)
        return FA_ERR_LAUNCH;
    fa::MergeParams mp;
    mp.ws_o = ws_o;
    mp.ws_lse = ws_lse;
    mp.o = o;
    mp.lse = lse;
    mp.rows = rows;
    mp.n_splits = s_last;
    mp.split_u = u;
    mp.N = N;
    mp.block_r = t.block_r;
    mp.n_qtiles = (int)n_qtiles;
    void* margs[] = {&mp};
    if (hipLaunchKernel(me->fn, dim3((unsigned)merge_grid), dim3(256), margs, 0, s) != hipSuccess)
        return FA_ERR_LAUNCH;
    return FA_OK;
}

}  // namespace fa

extern "C" {

int fa_tile_supported(int d, fa_dtype_t in_dtype, fa_dtype_t out_dtype, const fa_tile* tile) {
    const fa_tile t = resolve(1, 1, 1, d, in_dtype, 0, tile);  // NULL, {0, 0}: the base tile
    return find(d, t, in_dtype, out_dtype, 0, 0) ? FA_OK : FA_ERR_TILE;
}

int fa_default_tile(int B, int H, int N, int d, fa_dtype_t in_dtype, fa_dtype_t out_dtype, int causal,
                    int has_mask, fa_tile* out) {
    (void)has_mask;
    if (!out) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (!dtype_pair_ok(in_dtype, out_dtype)) return FA_ERR_DTYPE;
    *out = auto_tile(B, H, N, d, in_dtype, causal);
    return FA_OK;
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
              int d, float scale, int causal, const uint8_t* key_padding_mask, fa_dtype_t in_dtype,
              fa_dtype_t out_dtype, hipStream_t stream, const fa_tile* tile) {
    const int st = check_common(q, k, v, o, lse, B, H, N, d, scale, in_dtype, out_dtype);
    if (st != FA_OK) return st;
    const fa_tile t = resolve(B, H, N, d, in_dtype, causal, tile);
    if (t.block_r <= 0 || t.block_r % 32 != 0) return FA_ERR_TILE;
    // Sizes: every byte offset is computed in 64 bits on the device, but a
    // row index times the row size must fit in 32 bits, and so must the grid.
    const long long rows = (long long)B * H * N;
    const long long n_qtiles = ((long long)N + t.block_r - 1) / t.block_r;
    const long long grid = (long long)B * H * n_qtiles;
    if (rows > (1LL << 40) || (long long)N * d * 4 > INT32_MAX || grid > INT32_MAX) return FA_ERR_SHAPE;
    const Entry* e = find(d, t, in_dtype, out_dtype, causal, key_padding_mask != nullptr);
    if (!e) return FA_ERR_TILE;

    fa::Params prm;
    fill_params(prm, q, k, v, o, lse, key_padding_mask, B, H, N, scale, causal, n_qtiles, grid);
    // Causal 16-bit launches deal their query tiles in groups of four heads
    // when every XCD holds a multiple of four (B*H a multiple of 32): the
    // tail of the launch stays fuller than with pairs. Same process, causal
    // d = 128, N = 8192, 64 heads, 128 x 32, two cards: G = 4 0.9979-0.9984
    // ms against G = 2 1.0149-1.0237 (+1.7-2.6%), G = 8 1.0148, G = 1
    // 1.0604; for 256 x 64 G = 4 +0.4%. The K/V of four heads at once miss
    // the L2 more often (more fabric reads), which the launch absorbs.
    if (causal && in_dtype != FA_DTYPE_F32 && (long long)B * H % 32 == 0) prm.head_group = 4;
    // When every workgroup is resident from the start (the grid fits the 256
    // CUs at once) and all have the same work (no causal or key mask), the
    // launch ends when the slowest workgroup does. The SIMDs issue from the
    // oldest wave first, so one of the co-resident workgroups of each CU
    // finishes early and the other runs its last part alone (on the d = 64
    // non-causal workload: half the workgroups end at 54-59 us, half at
    // 76-81 us). Priorities that follow each wave's progress even this out
    // (+2% there); with a causal mask the oldest workgroups hold the longest
    // tiles and should finish first, so it stays off.
    const fa_tile dt = default_tile(d, in_dtype);
    prm.fair = (!causal && !key_padding_mask && t.block_r == dt.block_r && t.block_c == dt.block_c &&
                grid <= 256LL * resident_wgs_per_cu(d, in_dtype))
                   ? 1
                   : 0;
    void* args[] = {&prm};
    const hipError_t err = hipLaunchKernel(e->fn, dim3((unsigned)grid), dim3(e->nwaves * 64), args, 0,
                                           reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, const uint8_t* key_padding_mask, fa_dtype_t in_dtype, fa_dtype_t out_dtype,
           hipStream_t stream) {
    return fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask, in_dtype, out_dtype,
                     stream, nullptr);
}

size_t fa_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits) {
    return splitkv_bytes(B, H, N, d, num_splits);
}

int fa_splitkv_num_splits(int B, int H, int N, int d, fa_dtype_t in_dtype, int causal) {
    if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (in_dtype != FA_DTYPE_F32 && in_dtype != FA_DTYPE_BF16 && in_dtype != FA_DTYPE_F16) return FA_ERR_DTYPE;
    const fa_tile t = default_tile(d, in_dtype);
    const long long grid = (long long)B * H * (((long long)N + t.block_r - 1) / t.block_r);
    const long long key_tiles = ((long long)N + t.block_c - 1) / t.block_c;
    if (split_plan(B, H, N, d, in_dtype, causal, 1).u > 0) {
        // Causal parts in proportion to the keys: the smallest count whose
        // workgroups reach 9/16 of the slots, at most 12, with at least four
        // key tiles per part of the longest query tile. Same-card sweeps of
        // 2 .. 24 on causal d = 128, N = 8192: the best counts were 6 - 12
        // for 1 head (219 - 374 workgroups), 6 for 2 heads (438), 3 for 4
        // heads (504); more parts than that lost 10 - 25%.
        const long long target = 256LL * resident_wgs_per_cu(d, in_dtype) * 9 / 16;
        int s = 1;
        while (s < 12 && key_tiles / (s + 1) >= 4 &&
               (long long)B * H * split_plan(B, H, N, d, in_dtype, causal, s).parts < target)
            ++s;
        return s;
    }
    // Enough parts to fill every workgroup slot of the 256 CUs at once,
    // keeping at least four key tiles per part and at most 8 parts (beyond
    // that the merge, which reads every part's row, costs more than the
    // extra parallelism gains: 1 x 1 x 8192 runs 287 TFLOP/s at 8 parts and
    // 270 at 12). fp32 tiles run on the fp32 MFMA, many times slower per
    // tile, so one tile per part already outweighs the merge (the 1 x 1 x
    // 256 fp32 launch: 24 us unsplit, 16 us in 4 parts).
    const long long slots = 256LL * resident_wgs_per_cu(d, in_dtype);
    const long long min_tiles = in_dtype == FA_DTYPE_F32 ? 1 : 4;
    long long s = 1;
    while (s < 8 && grid * s < slots && key_tiles / (s + 1) >= min_tiles) ++s;
    return (int)s;
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                   int d, float scale, int causal, const uint8_t* key_padding_mask, fa_dtype_t in_dtype,
                   fa_dtype_t out_dtype, int num_splits, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
    const int st = fa::check_splitkv(q, k, v, o, lse, B, H, N, d, scale, in_dtype, out_dtype, num_splits);
    if (st != FA_OK) return st;
    const size_t need = splitkv_bytes(B, H, N, d, num_splits);
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return FA_ERR_WORKSPACE;
    return fa::launch_splitkv(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask, in_dtype, out_dtype,
                          num_splits, workspace, stream);
}

}  // extern "C"
