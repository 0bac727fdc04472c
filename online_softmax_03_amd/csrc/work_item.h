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

// Host side: G for a launch over n_heads heads. Without a causal mask every
// item has the same length and the order does not matter (G = 1). With one,
// G = 2 when every XCD's share of the grid holds an even number of heads
// (the shares hold n_heads / 8 heads each), so that no pair straddles two
// XCDs. Measured on the causal d = 128, N = 8192, 64-head launch: +2%
// throughput for 1.5x the HBM reads (K/V re-read from outside the L2 when
// two heads are streamed at once); G = 4 gained another 0-1% for 2-4x the
// reads.
constexpr int head_group_for(int n_heads, int causal) {
    return (causal && n_heads % 16 == 0) ? 2 : 1;
}

}  // namespace fa
