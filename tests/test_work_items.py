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


PARTS_DRIVER = r"""
#include <cstdio>
#include <vector>
#include "work_item.h"

// Causal split-KV parts: query tile qt of n_q (block_r rows) sees the key
// tiles of its causal extent; the parts of a launch whose longest tile gets
// at most S parts.
int main() {
    long cases = 0, bad = 0;
    const int shapes[][2] = {{128, 32}, {256, 64}, {128, 64}};  // block_r, block_c
    const int Ns[] = {1, 31, 32, 127, 128, 129, 200, 1000, 2048, 4095, 8192, 8193, 32768};
    const int Ss[] = {1, 2, 3, 4, 5, 7, 8, 12, 16, 24, 64};
    const int heads[] = {1, 2, 3, 8, 16};
    for (auto& sh : shapes)
        for (int N : Ns)
            for (int S : Ss) {
                const int BR = sh[0], BC = sh[1], r = BR / BC;
                const int n_q = (N + BR - 1) / BR, n_k = (N + BC - 1) / BC;
                const int u = fa::split_unit(n_k, r, S);
                const int s_last = (n_k + u * r - 1) / (u * r);
                const long long P = fa::parts_per_head(n_q, u, s_last);
                bool ok = u >= 1 && s_last >= 1 && s_last <= S;
                long long sum = 0;
                for (int qt = 0; qt < n_q && ok; ++qt) {
                    const int np = fa::parts_of(qt, n_q, u, s_last);
                    if (fa::parts_before(qt, u) != sum && qt < n_q) { printf("parts_before qt=%d\n", qt); ok = false; }
                    sum += np;
                    // every part of the causal extent holds at most u*r key tiles
                    const int ext = (qt == n_q - 1 ? N : (qt + 1) * BR);
                    const int nt = (ext + BC - 1) / BC;
                    const int per = (nt + np - 1) / np;
                    if (np < 1 || np > s_last || per > u * r) { printf("parts BR=%d BC=%d N=%d S=%d qt=%d np=%d per=%d\n", BR, BC, N, S, qt, np, per); ok = false; }
                }
                if (ok && sum != P) { printf("P BR=%d N=%d S=%d\n", BR, N, S); ok = false; }
                // the longest tile's part length is what S asks for, no coarser
                if (ok && n_k >= S && u * r > r * (((n_k + S - 1) / S + r - 1) / r)) { printf("u too large\n"); ok = false; }
                for (int H : heads) {
                    if (!ok) break;
                    const long long grid = (long long)H * P;
                    const int mode = fa::xcd_mode_for(H, grid);
                    std::vector<int> seen((size_t)H * n_q * S, 0);
                    std::vector<int> prev_qt((size_t)H, n_q);
                    for (long long b = 0; b < grid && ok; ++b) {
                        int bh = -1, qt = -1, s = -1;
                        long long k = -1;
                        fa::schedule_parts((int)b, (int)grid, P, mode, &bh, &k);
                        if (bh < 0 || bh >= H || k < 0 || k >= P) { printf("range b=%lld\n", b); ok = false; break; }
                        fa::locate_part(k, n_q, u, s_last, &qt, &s);
                        if (qt < 0 || qt >= n_q || s < 0 || s >= fa::parts_of(qt, n_q, u, s_last)) { printf("locate k=%lld\n", k); ok = false; break; }
                        ++seen[((size_t)bh * n_q + qt) * S + s];
                        if (mode == fa::kXcdHeads && bh % 8 != (int)(b % 8)) { printf("head %d on XCD %lld\n", bh, b % 8); ok = false; }
                        // each head's parts run from the last query tile to the first
                        if (mode != fa::kXcdChunks) {
                            if (qt > prev_qt[(size_t)bh]) { printf("order H=%d N=%d S=%d\n", H, N, S); ok = false; }
                            prev_qt[(size_t)bh] = qt;
                        }
                    }
                    long long used = 0;
                    for (size_t i = 0; i < seen.size() && ok; ++i) {
                        if (seen[i] > 1) { printf("part twice H=%d N=%d S=%d\n", H, N, S); ok = false; }
                        used += seen[i];
                    }
                    if (ok && used != grid) { printf("not every part H=%d N=%d S=%d\n", H, N, S); ok = false; }
                    ++cases;
                }
                if (!ok) ++bad;
            }
    printf("%ld cases, %ld bad\n", cases, bad);
    return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_causal_split_parts_cover_every_part_once(tmp_path):
    """Causal split-KV launches: every (head, query tile, part) with part <
    parts_of(tile) is one workgroup, no part holds more than u*r key tiles of
    its tile's causal extent, the longest tile has at most the requested
    count, and each head's parts run from the last query tile to the first."""
    src = tmp_path / "parts.cpp"
    src.write_text(PARTS_DRIVER)
    exe = tmp_path / "parts"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr
    assert " 0 bad" in r.stdout
