// Merge of split-KV partial results on gfx950.
//
// Part s of a row covers a contiguous range of keys and delivers its
// normalised output O_s and LSE_s = m_s + ln l_s. Two partial states combine
// as m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m), O likewise (the merge
// equations of the online-softmax interview card, section 三, associative by
// "La recurrencia del online softmax", practice problem 4). In LSE form, with
// M = max_s LSE_s and w_s = e^(LSE_s - M):
//
//   O = sum_s w_s O_s / sum_s w_s,   LSE = M + ln sum_s w_s,
//
// and a row whose parts are all empty (every LSE_s = -inf) gets O = 0 and
// LSE = -inf. Each thread owns four consecutive d values of one row; the
// kernel streams the partials once, so it is bound by HBM bandwidth.
#pragma once

#include "attn_common.h"

namespace fa {

struct MergeParams {
    const float* ws_o;    // [n_splits][rows][d]
    const float* ws_lse;  // [n_splits][rows]
    void* o;              // [rows][d] of the output dtype
    float* lse;           // [rows]
    long long rows;       // B * H * N
    int n_splits;
    // causal split launches (split_u > 0): the row's query tile (rows of N
    // per head, block_r per tile, n_qtiles per head) has parts_of(...) parts
    int split_u;
    int N, block_r, n_qtiles;
};

constexpr float kLog2e = 1.44269504088896340736f;

template <int D, typename TO>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams mp) {
    constexpr int TPR = D / 4;          // threads per row
    constexpr int RPB = 256 / TPR;      // rows per block
    const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int t = threadIdx.x % TPR;
    if (row >= mp.rows) return;
    const int S = mp.split_u > 0
                      ? parts_of((int)(row % mp.N) / mp.block_r, mp.n_qtiles, mp.split_u, mp.n_splits)
                      : mp.n_splits;
    // Parts in groups of kGroup whose loads are all issued before the first
    // is used, instead of a loop that waits for each part's load in turn (at
    // B*H = 1, N = 8192, about 6 parts per row: 9.3 -> 7.0 us; groups of 8
    // took more registers and were slower with 2 parts per row); the
    // additions keep the order s = 0, 1, ..., S - 1.
    constexpr int kGroup = 4;
    float M = -INFINITY;
    for (int s0 = 0; s0 < S; s0 += kGroup) {
        float l[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i)
            l[i] = s0 + i < S ? mp.ws_lse[(long long)(s0 + i) * mp.rows + row] : -INFINITY;
#pragma unroll
        for (int i = 0; i < kGroup; ++i) M = fmaxf(M, l[i]);
    }
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    float out_lse = -INFINITY;
    float inv = 0.f;
    if (M != -INFINITY) {
        float L = 0.f;
        for (int s0 = 0; s0 < S; s0 += kGroup) {
            float l[kGroup];
            f32x4 x[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const long long pr = (long long)(s0 + i) * mp.rows + row;
                if (s0 + i < S) {
                    l[i] = mp.ws_lse[pr];
                    x[i] = *reinterpret_cast<const f32x4*>(mp.ws_o + pr * D + 4 * t);
                }
            }
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                if (s0 + i < S) {
                    const float w = __builtin_amdgcn_exp2f((l[i] - M) * kLog2e);  // e^(LSE_s - M)
                    L += w;
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = __builtin_fmaf(w, x[i][j], o[j]);
                }
            }
        }
        inv = 1.f / L;
        out_lse = M + __builtin_amdgcn_logf(L) / kLog2e;  // ln L = log2 L / log2 e
    }
    char* orow = reinterpret_cast<char*>(mp.o) + (row * D + 4 * t) * TO::kBytes;
    store_row4<TO>(orow, o, inv);
    if (t == 0) mp.lse[row] = out_lse;
}

}  // namespace fa
