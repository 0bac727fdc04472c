"""The work-item order of the attention kernels (CPU; the header is plain
constexpr C++ and is compiled here with g++).

Every launch maps workgroup ids onto (key-range part, batch*head, tile)
through `schedule`, which spreads the heads over the 8 XCDs and orders each
XCD's items with `work_item`; the checks below run those same functions over
many shapes, part counts, group sizes and XCD modes: every id must land on a
distinct triple in range (a bijection), tiles must be dealt from the last to
the first within every group, the head mode must keep every head on the one
XCD its index names, and the host's choices (group size, XCD mode) must fit
the shape.
"""
import os
import shutil
import subprocess

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "online_softmax_03_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <vector>
#include "work_item.h"

int main() {
    long cases = 0, bad = 0;
    const int heads[] = {1, 2, 3, 5, 7, 8, 12, 15, 16, 24, 32, 40, 48, 64, 96, 128, 200};
    const int tiles[] = {1, 2, 3, 5, 63, 64, 65, 256};
    const int groups[] = {-1, 0, 1, 2, 3, 4, 5, 8, 16, 100, 1000};
    for (int H : heads)
        for (int nt : tiles)
            for (int G : groups) {
                std::vector<int> seen((size_t)H * nt, 0);
                int prev_tile = nt;  // tiles never grow within a group
                int prev_grp = -1;
                const int g = G < 1 ? 1 : G;
                for (int id = 0; id < H * nt; ++id) {
                    int bh = -1, t = -1;
                    fa::work_item(id, nt, H, G, &bh, &t);
                    if (bh < 0 || bh >= H || t < 0 || t >= nt) { ++bad; printf("range H=%d nt=%d G=%d id=%d\n", H, nt, G, id); break; }
                    ++seen[(size_t)bh * nt + t];
                    const int grp = bh / g;
                    if (grp != prev_grp) { prev_grp = grp; prev_tile = nt; }
                    if (t > prev_tile) { ++bad; printf("order H=%d nt=%d G=%d id=%d\n", H, nt, G, id); break; }
                    prev_tile = t;
                }
                for (int c : seen)
                    if (c != 1) { ++bad; printf("not a bijection H=%d nt=%d G=%d\n", H, nt, G); break; }
                ++cases;
            }
    // the launch's group size: 1 without a causal mask; with one, a divisor of
    // every XCD share (n_heads / 8 heads) when it is above 1
    for (int H = 1; H <= 512; ++H)
        for (int causal = 0; causal < 2; ++causal) {
            const int g = fa::head_group_for(H, causal);
            if (g < 1 || (!causal && g != 1) || (g > 1 && (H % 8 != 0 || (H / 8) % g != 0))) {
                ++bad; printf("group H=%d causal=%d -> %d\n", H, causal, g);
            }
            ++cases;
        }
    // G = 1 is the plain order: head after head, last tile first
    for (int id = 0; id < 7 * 5; ++id) {
        int bh, t;
        fa::work_item(id, 5, 7, 1, &bh, &t);
        if (bh != id / 5 || t != 4 - id % 5) { ++bad; printf("G=1 id=%d\n", id); }
    }
    // G = 2 interleaves pairs: ids 0,1 are the last tiles of heads 0 and 1
    int b0, t0, b1, t1, b2, t2;
    fa::work_item(0, 4, 4, 2, &b0, &t0);
    fa::work_item(1, 4, 4, 2, &b1, &t1);
    fa::work_item(2, 4, 4, 2, &b2, &t2);
    if (!(b0 == 0 && t0 == 3 && b1 == 1 && t1 == 3 && b2 == 0 && t2 == 2)) { ++bad; printf("G=2 order\n"); }
    // schedule: every XCD mode the host can pick, with key-range parts
    const int splits[] = {1, 2, 3, 8};
    for (int H : heads)
        for (int nt : tiles)
            for (int S : splits)
                for (int G : {1, 2, 4})
                    for (int mode = 0; mode < 3; ++mode) {
                        const long long grid = (long long)H * nt * S;
                        if (grid > 200000) continue;
                        if (mode == fa::kXcdHeads && H % 8 != 0) continue;
                        if (mode == fa::kXcdChunks && grid % 8 != 0) continue;
                        std::vector<int> seen((size_t)grid, 0);
                        std::vector<int> xcd_of_head((size_t)H, -1);
                        bool ok = true;
                        for (int b = 0; b < grid && ok; ++b) {
                            int sp = -1, bh = -1, t = -1;
                            fa::schedule(b, (int)grid, nt, H, S, G, mode, &sp, &bh, &t);
                            if (sp < 0 || sp >= S || bh < 0 || bh >= H || t < 0 || t >= nt) {
                                printf("schedule range H=%d nt=%d S=%d G=%d mode=%d b=%d\n", H, nt, S, G, mode, b);
                                ok = false;
                                break;
                            }
                            ++seen[((size_t)bh * nt + t) * S + sp];
                            if (mode == fa::kXcdHeads) {
                                // XCD b % 8 runs whole heads, those with bh % 8 == b % 8
                                if (bh % 8 != b % 8) { printf("head %d on XCD %d\n", bh, b % 8); ok = false; }
                            }
                            if (mode != fa::kXcdNone) {
                                int& x = xcd_of_head[(size_t)bh];
                                if (mode == fa::kXcdHeads && x >= 0 && x != b % 8) { printf("head split over XCDs\n"); ok = false; }
                                x = b % 8;
                            }
                        }
                        for (int c : seen)
                            if (ok && c != 1) { printf("schedule not a bijection H=%d nt=%d S=%d G=%d mode=%d\n", H, nt, S, G, mode); ok = false; }
                        if (!ok) ++bad;
                        ++cases;
                    }
    // the host's choice: heads mode exactly when the heads divide over the XCDs
    for (int H = 1; H <= 64; ++H)
        for (long long grid : {8LL, 12LL, 64LL})
            if ((fa::xcd_mode_for(H, grid) == fa::kXcdHeads) != (H % 8 == 0) ||
                (H % 8 != 0 && (fa::xcd_mode_for(H, grid) == fa::kXcdChunks) != (grid % 8 == 0))) {
                ++bad;
                printf("xcd_mode_for H=%d grid=%lld\n", H, grid);
            }
    printf("%ld cases, %ld bad\n", cases, bad);
    return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_schedule_is_a_bijection_in_heavy_first_order(tmp_path):
    src = tmp_path / "wi.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "wi"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 bad" in r.stdout
