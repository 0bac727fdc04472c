// Attention forward with online softmax for fp32 inputs on gfx950.
//
// The same tiled loop as the 16-bit kernel (see attn_fwd_kernel.h for the
// step-by-step description and the pages it follows), with both products on
// v_mfma_f32_32x32x2_f32 and P kept in fp32, so nothing is rounded below
// fp32. It is not software-pipelined: fp32 inputs only serve small problems.
//
//   S^T = K_j Q^T: instruction t of a 32x32 block contracts the d pair
//     (t, D/2 + t): lane (col, hh) supplies K[key][hh*D/2 + t] and
//     Q[query][hh*D/2 + t].
//   O^T += V_j^T P^T: register r of the S^T block is key 8(r/4) + 4*hh + r%4,
//     the k = hh slot of instruction r, whose A operand is V[that key][d].
#pragma once

#include "attn_common.h"

namespace fa {

template <int D, int BC, int NW, bool CAUSAL, bool MASK, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void attn_fwd_f32_kernel(Params p) {
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BC % 32 == 0 && BC >= 32 && BC <= 64, "key tile");
    constexpr int NT = NW * 64;
    constexpr int BR = NW * 32;
    constexpr int NKB = BC / 32;
    constexpr int NDB = D / 32;
    constexpr int ROWB = D * 4;
    constexpr int CH = ROWB / 16;
    constexpr int TILEB = BC * ROWB;
    constexpr int RPI = 1024 / ROWB;
    constexpr int LOADS = TILEB / 1024;
    constexpr int LPW = (LOADS + NW - 1) / NW;

    __shared__ __attribute__((aligned(1024))) char buf0[2 * TILEB];
    __shared__ __attribute__((aligned(1024))) char buf1[2 * TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int hh = lane >> 5;

    int split, n_parts, bh, qt;
    attn_schedule<SPLIT, CAUSAL>(p, &split, &n_parts, &bh, &qt);
    const int b = bh / p.H;
    const int N = p.N;
    const int q0 = qt * BR;
    const int qw0 = q0 + wave * 32;

    const size_t head = (size_t)bh * (size_t)N * D;
    const char* qg = reinterpret_cast<const char*>(p.q) + head * 4;
    const char* kg = reinterpret_cast<const char*>(p.k) + head * 4;
    const char* vg = reinterpret_cast<const char*>(p.v) + head * 4;

    int key_lo = 0, key_hi = N;
    bool mask_general = false;
    const uint8_t* mrow = MASK ? p.mask + (size_t)b * N : nullptr;
    if constexpr (MASK) {
        int first, last, count;
        mask_extent<NT>(mrow, N, &first, &last, &count);
        if (last < 0) {
            key_hi = 0;
        } else {
            key_lo = first;
            key_hi = last + 1;
            mask_general = count != key_hi - key_lo;
        }
    }
    int kv_begin = (key_lo / BC) * BC;
    const int kv_end = CAUSAL ? min(key_hi, q0 + BR) : key_hi;
    int n_tiles = kv_end > kv_begin ? (kv_end - kv_begin + BC - 1) / BC : 0;
    if constexpr (SPLIT) {
        // this workgroup's part of the key tiles: [t0, t1) of n_tiles
        const int per = (n_tiles + n_parts - 1) / n_parts;
        const int t0 = min(n_tiles, split * per);
        const int t1 = min(n_tiles, t0 + per);
        kv_begin += t0 * BC;
        n_tiles = t1 - t0;
    }

    {
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int off = tid * 16; off < TILEB; off += NT * 16) {
            *reinterpret_cast<FA_LDS u32x4*>((FA_LDS char*)buf0 + TILEB + off) = z;
            *reinterpret_cast<FA_LDS u32x4*>((FA_LDS char*)buf1 + TILEB + off) = z;
        }
        __syncthreads();
    }

    u32 lane_off[LPW];
#pragma unroll
    for (int ii = 0; ii < LPW; ++ii) {
        const int R = wave + ii * NW;
        const int trow = R * RPI + lane / CH;
        lane_off[ii] = (u32)(trow * ROWB + (((lane % CH) ^ swz<CH>(trow)) * 16));
    }
    auto issue_tile = [&](int tile, char* buf) {
        const int k0 = kv_begin + tile * BC;
        const int bytes = (N - k0) * ROWB;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)(kg + (size_t)k0 * ROWB), 0, bytes, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)(vg + (size_t)k0 * ROWB), 0, bytes, kBufferFlags);
#pragma unroll
        for (int ii = 0; ii < LPW; ++ii) {
            const int R = wave + ii * NW;
            if (LOADS % NW != 0 && R >= LOADS) break;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FA_LDS void*)(buf + R * 1024), 16, lane_off[ii],
                                                     0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (FA_LDS void*)(buf + TILEB + R * 1024), 16,
                                                     lane_off[ii], 0, 0, 0);
        }
    };

    float qf[D / 2];
    {
        const int qr = min(qw0 + col, N - 1);
        const char* src = qg + (size_t)qr * ROWB + hh * (ROWB / 2);
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(src + i * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) qf[4 * i + j] = x[j];
        }
    }

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;
    const float c = p.c;
    const bool wave_live = qw0 < N;
    const int qq = qw0 + col;
    const int sw_col = swz<CH>(col);

    auto compute_tile = [&](int tile, const char* buf) {
        const int k0 = kv_begin + tile * BC;
        if (!wave_live || (CAUSAL && k0 > qw0 + 31)) return;
        const FA_LDS char* kt = (const FA_LDS char*)buf;
        const FA_LDS char* vt = (const FA_LDS char*)buf + TILEB;

        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int chunk = (hh * (D / 8) + i) ^ sw_col;
                const f32x4 a4 =
                    *reinterpret_cast<const FA_LDS f32x4*>(kt + (kb * 32 + col) * ROWB + chunk * 16);
#pragma unroll
                for (int j = 0; j < 4; ++j) s[kb] = mfma32x32x2_f32(a4[j], qf[4 * i + j], s[kb]);
            }
        }

        const bool edge_lo = k0 < key_lo;
        const bool edge_hi = k0 + BC > kv_end;
        const bool diag = CAUSAL && (k0 + BC - 1 > qw0);
        if (edge_lo || edge_hi || diag || (MASK && mask_general)) {
            const int base = k0 + 4 * hh;
            int hi = min(key_hi, kv_end) - 1 - base;
            if (CAUSAL) hi = min(hi, qq - base);
            const int lo = key_lo - base;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rel = kb * 32 + 8 * (r >> 2) + (r & 3);
                    bool ok = rel <= hi && rel >= lo;
                    if (MASK && mask_general) ok = ok && mrow[min(base + rel, N - 1)] != 0;
                    s[kb][r] = ok ? s[kb][r] : -INFINITY;
                }
            }
        }

        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = pair_max(mx);
        const float m_new = fmaxf(m_run, mx);
        if (__builtin_amdgcn_ballot_w64((m_new - m_run) * c > kRescaleLog2) != 0) {
            const float alpha =
                __builtin_amdgcn_exp2f(m_run * c - ((m_new == -INFINITY) ? 0.f : m_new * c));
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
            m_run = m_new;
        }
        const float ref = (m_run == -INFINITY) ? 0.f : m_run * c;
        // two chains for the row sum, each started from its first term
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -ref));
                float& rs = (r & 1) ? rs1 : rs0;
                rs = (kb == 0 && r < 2) ? s[kb][r] : rs + s[kb][r];
            }
        l_run += rs0 + rs1;

#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int chunk = (8 * db + (col >> 2)) ^ swz<CH>(key);
                    const float a = *reinterpret_cast<const FA_LDS float*>(vt + key * ROWB + chunk * 16 +
                                                                           (col & 3) * 4);
                    acc[db] = mfma32x32x2_f32(a, s[kb][r], acc[db]);
                }
            }
        }
    };

    if (n_tiles > 0) issue_tile(0, buf0);
    for (int it = 0; it < n_tiles; it += 2) {
        wait_vmcnt0();
        __syncthreads();
        if (it + 1 < n_tiles) issue_tile(it + 1, buf1);
        compute_tile(it, buf0);
        if (it + 1 >= n_tiles) break;
        wait_vmcnt0();
        __syncthreads();
        if (it + 2 < n_tiles) issue_tile(it + 2, buf0);
        compute_tile(it + 1, buf1);
    }

    const float l_tot = pair_sum(l_run);
    const bool dead = !(l_tot > 0.f);
    const float inv = dead ? 0.f : 1.f / l_tot;
    const float lse = dead ? -INFINITY : (m_run * c + __builtin_amdgcn_logf(l_tot)) * kLn2;
    if (SPLIT && qq < N) {
        // normalised partial output and LSE of this part of the keys
        const size_t prow = ((size_t)split * p.B * p.H + bh) * N + qq;
        char* orow = reinterpret_cast<char*>(p.ws_o + prow * D);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * db + 8 * g + 4 * hh;
                const float v4[4] = {acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2],
                                     acc[db][4 * g + 3]};
                store_row4<F32>(orow + d0 * 4, v4, inv);
            }
        if (hh == 0) p.ws_lse[prow] = lse;
    } else if (qq < N) {
        char* orow = reinterpret_cast<char*>(p.o) + (head + (size_t)qq * D) * 4;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * db + 8 * g + 4 * hh;
                const float v4[4] = {acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2],
                                     acc[db][4 * g + 3]};
                store_row4<F32>(orow + d0 * 4, v4, inv);
            }
        if (hh == 0) p.lse[(size_t)bh * N + qq] = lse;
    }
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace fa
