// Order in which the attention kernels take their work items (one workgroup
// per item: one query tile, or one key tile for the dK/dV kernel, of one
// batch*head). Plain constexpr code, so the same functions run on the host
// (tests) and on the device (clang compiles constexpr functions for both).
#pragma once

namespace fa {

// Item `id` (after the XCD remap) -> (batch*head `bh`, tile `tile`). The
// n_heads = B*H heads are taken in groups of G consecutive heads; inside a
// group the items run through the tiles from the last (n_tiles - 1) to the
// first and, for each tile, through the group's heads. The hardware starts
// workgroups in id order, so on each XCD the longest items (under a causal
// mask the last query tile has the most keys) start first. With G = 1 the
// last head of an XCD's share has its longest items start behind the short
// items of the head before it and the launch ends on a tail of idle
// workgroup slots; G = 2 interleaves pairs of heads. The last group may hold
// fewer than G heads; G < 1 counts as 1. Every id in [0, n_heads*n_tiles)
// maps to a distinct pair in [0, n_heads) x [0, n_tiles).
constexpr void work_item(int id, int n_tiles, int n_heads, int G, int* bh, int* tile) {
    if (G < 1) G = 1;
    const int grp = id / (G * n_tiles);
    const int r = id - grp * G * n_tiles;
    const int left = n_heads - grp * G;
    const int gh = G < left ? G : left;
    const int t = r / gh;
    *bh = grp * G + (r - t * gh);
    *tile = n_tiles - 1 - t;
}

// How workgroup ids are spread over the 8 XCDs. The hardware deals
// workgroup ids round-robin: id b runs on XCD b % 8, and each XCD starts its
// ids in increasing order.
//   kXcdHeads (B*H a multiple of 8): XCD x takes heads x, x + 8, x + 16, ...
//     whole (every tile of a head on one XCD, so its K and V are read into
//     one L2), and heads of every batch alike, so work that differs by batch
//     (key-padding lengths) is spread evenly over the XCDs.
//   kXcdChunks (grid a multiple of 8 only): XCD x takes the x-th eighth of
//     the items in head-major order (parts of at most two heads).
//   kXcdNone: the ids as they come.
enum XcdMode { kXcdNone = 0, kXcdChunks = 1, kXcdHeads = 2 };

// Workgroup `block` of a grid of n_heads * n_tiles * n_splits -> (key-range
// part `split`, batch*head `bh`, tile `tile`), by the XCD mode above and, on
// each XCD, by work_item over that XCD's heads (group size G). Every block
// in [0, grid) maps to a distinct triple; the split part varies fastest, so
// the parts of one tile run side by side.
constexpr void schedule(int block, int grid, int n_tiles, int n_heads, int n_splits, int G, int xcd_mode,
                        int* split, int* bh, int* tile) {
    if (xcd_mode == kXcdHeads) {
        const int x = block & 7;
        int k = block >> 3;
        *split = k % n_splits;
        k /= n_splits;
        int j = 0;
        work_item(k, n_tiles, n_heads / 8, G, &j, tile);
        *bh = j * 8 + x;
        return;
    }
    int id = block;
    if (xcd_mode == kXcdChunks) id = (block & 7) * (grid >> 3) + (block >> 3);
    *split = id % n_splits;
    id /= n_splits;
    work_item(id, n_tiles, n_heads, G, bh, tile);
}

// Split-KV parts under a causal mask. Query tile qt of n_q (B_r rows each)
// sees r*(qt+1) key tiles of B_c keys (r = B_r / B_c), the last one all n_k
// of them, so equal part counts per query tile would give the parts of the
// last tiles the most keys and the launch would wait for them. Instead each
// part gets at most u*r key tiles: query tile qt < n_q - 1 has
// ceil((qt+1)/u) parts and the last one s_last = ceil(n_k / (u*r)), the
// most of any tile (the caller's part count). parts_of gives a tile's
// count, parts_before the sum over the tiles before it,
// sum_{j=1..qt} ceil(j/u) = u*Q*(Q+1)/2 + R*(Q+1) with qt = Q*u + R.
constexpr int parts_of(int qt, int n_q, int u, int s_last) {
    return qt < n_q - 1 ? (qt + u) / u : s_last;
}

constexpr long long parts_before(int qt, int u) {
    const long long Q = qt / u, R = qt - Q * u;
    return (long long)u * Q * (Q + 1) / 2 + R * (Q + 1);
}

constexpr long long parts_per_head(int n_q, int u, int s_last) { return parts_before(n_q - 1, u) + s_last; }

// Part k of a head (0 <= k < parts_per_head) -> query tile `qt` and its part
// `s`, by a binary search over parts_before (increasing in qt).
constexpr void locate_part(long long k, int n_q, int u, int s_last, int* qt, int* s) {
    const long long last0 = parts_before(n_q - 1, u);
    if (k >= last0) {
        *qt = n_q - 1;
        *s = (int)(k - last0);
        return;
    }
    int lo = 0, hi = n_q - 2;  // the largest q with parts_before(q) <= k
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (parts_before(mid, u) <= k) lo = mid;
        else hi = mid - 1;
    }
    *qt = lo;
    *s = (int)(k - parts_before(lo, u));
}

// Workgroup `block` of a causal split launch (n_heads * P workgroups, P =
// parts_per_head) -> (batch*head `bh`, part `k` of that head), by the XCD
// modes above; each head's parts run from the last (those of the last query
// tile) to the first.
constexpr void schedule_parts(int block, int grid, long long P, int xcd_mode, int* bh, long long* k) {
    long long id = 0;
    if (xcd_mode == kXcdHeads) {
        const long long j = block >> 3;  // the j-th item of XCD block % 8
        *bh = (int)(j / P) * 8 + (block & 7);
        id = j % P;
    } else {
        long long b = block;
        if (xcd_mode == kXcdChunks) b = (long long)(block & 7) * (grid >> 3) + (block >> 3);
        *bh = (int)(b / P);
        id = b % P;
    }
    *k = P - 1 - id;
}

// Host side: u for a causal split launch whose longest query tile (n_k key
// tiles) gets at most `num_splits` parts, r = B_r / B_c: the smallest u with
// ceil(n_k / (u*r)) <= num_splits.
constexpr int split_unit(int n_k, int r, int num_splits) {
    const int per = (n_k + num_splits - 1) / num_splits;  // key tiles per part, at least
    const int u = (per + r - 1) / r;
    return u < 1 ? 1 : u;
}

// Host side: the XCD mode of a launch over n_heads heads and `grid`
// workgroups.
constexpr int xcd_mode_for(int n_heads, long long grid) {
    return n_heads % 8 == 0 ? kXcdHeads : (grid % 8 == 0 ? kXcdChunks : kXcdNone);
}

// Host side: G for a launch over n_heads heads. Without a causal mask every
// item has the same length and the order does not matter (G = 1). With one,
// G = 2 when every XCD holds an even number of heads (n_heads / 8 each under
// kXcdHeads). Measured on the causal d = 128, N = 8192, 64-head launch: +2%
// throughput for 1.5x the HBM reads (K/V re-read from outside the L2 when
// two heads are streamed at once); G = 4 gained another 0-1% for 2-4x the
// reads.
constexpr int head_group_for(int n_heads, int causal) {
    return (causal && n_heads % 16 == 0) ? 2 : 1;
}

}  // namespace fa
