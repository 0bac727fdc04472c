// Attention backward from the saved LSE for gfx950 (MI355X), bf16/fp16 inputs.
//
// The forward keeps no N x N matrix, so the backward recomputes the scores
// S = scale * Q K^T tile by tile and recovers the probabilities directly
// from the row's LSE, P = exp(S - LSE), without another online pass
// ("Online Softmax 算法详解" section 8.3; the online-softmax interview card,
// section 四, point ③). With D_i = sum_t dO_it O_it the gradients are
//
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,
//   dK = scale dS^T Q,
//
// the chain rule through P V and through the row softmax. Three kernels, on
// the caller's stream in this order (at d = 64 the last two run as one
// launch, attn_bwd_fused_kernel below):
//
//   attn_bwd_prep_kernel  D_i and LSE_i * log2(e) for every query, written to
//     a workspace laid out in groups of 32 queries, [lse2 x 32][D x 32] per
//     group, padded to a multiple of 64 queries with lse2 = +inf and D = 0 (so
//     padded and fully masked rows give P = 2^-inf = 0 with no extra test).
//   attn_bwd_dq_kernel    one workgroup per query tile, walking the key tiles
//     as the forward does: S^T = K Q^T and dP^T = V dO^T with one query per
//     lane, P^T and dS^T in registers, dQ^T += K^T dS^T with K^T read from the
//     row-major K tile by ds_read_b64_tr_b16 and dS^T fed back as the B
//     operand (the forward's P V step with K in place of V).
//   attn_bwd_dkdv_kernel  one workgroup per key tile, walking the query
//     tiles: V of the wave's 32 keys stays in registers and K in LDS (loaded
//     once), Q, dO and the tile's (lse2, D) stream through LDS; S = Q K^T and
//     dP = dO V^T with one key per lane, dV^T += dO^T P and dK^T += Q^T dS
//     with dO^T and Q^T read by the transpose loads.
//
// No atomics: each gradient element is accumulated by exactly one lane in
// fp32 registers and stored once, so results are deterministic. P and dS are
// rounded to bf16/fp16 only as MFMA operands.
#pragma once

#include "attn_common.h"

namespace fa {

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;      // [B][H][N] natural log, from the forward
    float* stats;          // workspace: [B*H][n_g][lse2 x 32, D x 32]
    void* dq;
    void* dk;
    void* dv;
    const uint8_t* mask;   // [B][N] or nullptr
    int B, H, N;
    int n_g;               // 32-query groups per head, padded to an even count
    int n_qtiles;          // dQ kernel: ceil(N / B_r)
    int n_ktiles;          // dK/dV kernel: ceil(N / B_k)
    int xcd_remap;         // XcdMode: how workgroup ids spread over the 8 XCDs
    int head_group;        // heads whose tiles are dealt together (>= 1)
    int n_dkdv_blocks;     // fused kernel: workgroups [0, n) are dK/dV, the rest dQ
    float c;               // scale * log2(e)
    float scale;
};

constexpr float kBwdLog2e = 1.44269504088896340736f;

// ---------------------------------------------------------------- prep

// D/8 lanes per row (one 16-byte vector each); rows cover the padded groups.
template <int D, typename TI>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int TPR = D / 8;
    constexpr int RPB = 256 / TPR;
    const long long slot = (long long)blockIdx.x * RPB + threadIdx.x / TPR;  // padded query row
    const int t = threadIdx.x % TPR;
    const long long per_head = (long long)p.n_g * 32;
    const long long total = (long long)p.B * p.H * per_head;
    const bool in_range = slot < total;
    const long long bh = in_range ? slot / per_head : 0;
    const int q = in_range ? (int)(slot - bh * per_head) : 0;
    const bool live = in_range && q < p.N;
    float acc = 0.f;
    if (live) {
        const size_t off = ((size_t)bh * p.N + q) * D + 8 * t;
        const char* orow = reinterpret_cast<const char*>(p.o) + off * TI::kBytes;
        const char* drow = reinterpret_cast<const char*>(p.dout) + off * TI::kBytes;
        float a8[8], g8[8];
        if constexpr (__is_same(TI, BF16)) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(orow);
            const u32x4 g = *reinterpret_cast<const u32x4*>(drow);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a8[2 * i] = __uint_as_float(a[i] << 16);
                a8[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
                g8[2 * i] = __uint_as_float(g[i] << 16);
                g8[2 * i + 1] = __uint_as_float(g[i] & 0xffff0000u);
            }
        } else {
            const f16x8 a = *reinterpret_cast<const f16x8*>(orow);
            const f16x8 g = *reinterpret_cast<const f16x8*>(drow);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                a8[i] = (float)a[i];
                g8[i] = (float)g[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(a8[i], g8[i], acc);
    }
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (in_range && t == 0) {
        float lse2 = INFINITY;  // padded rows and rows with no allowed key: P = 0
        if (live) {
            const float l = p.lse[(size_t)bh * p.N + q];
            lse2 = (l == -INFINITY) ? INFINITY : l * kBwdLog2e;
        }
        float* grp = p.stats + ((size_t)bh * p.n_g + q / 32) * 64;
        grp[q % 32] = lse2;
        grp[32 + q % 32] = live ? acc : 0.f;
    }
#endif
}

// ---------------------------------------------------------------- dQ

// The body takes its workgroup index and the number of workgroups that share
// the work (the dQ kernel's grid, or its part of the fused grid below).
template <int D, int BC, int NW, typename TI, typename TO, bool CAUSAL, bool MASK>
__device__ __forceinline__ void bwd_dq_body(const BwdParams& p, int block, int grid) {
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BC % 32 == 0 && BC >= 32 && BC <= 64, "key tile");
    static_assert(TI::kBytes == 2, "16-bit inputs");
    constexpr int NT = NW * 64;
    constexpr int BR = NW * 32;
    constexpr int NKB = BC / 32;
    constexpr int NDC = D / 16;
    constexpr int NDB = D / 32;
    constexpr int EB = 2;
    constexpr int ROWB = D * EB;
    constexpr int CH = ROWB / 16;
    constexpr int TILEB = BC * ROWB;
    constexpr int RPI = 1024 / ROWB;
    constexpr int LOADS = TILEB / 1024;
    constexpr int LPW = (LOADS + NW - 1) / NW;

    // Two tile buffers, each K then V (distinct objects, see the forward).
    __shared__ __attribute__((aligned(1024))) char buf0[2 * TILEB];
    __shared__ __attribute__((aligned(1024))) char buf1[2 * TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int hh = lane >> 5;

    int split, bh, qt;  // workgroup -> (one key range, batch*head, query tile), as in the forward
    schedule(block, grid, p.n_qtiles, p.B * p.H, 1, p.head_group, p.xcd_remap, &split, &bh, &qt);
    const int b = bh / p.H;
    const int N = p.N;
    const int q0 = qt * BR;
    const int qw0 = q0 + wave * 32;

    const size_t head = (size_t)bh * (size_t)N * D;
    const char* qg = reinterpret_cast<const char*>(p.q) + head * EB;
    const char* kg = reinterpret_cast<const char*>(p.k) + head * EB;
    const char* vg = reinterpret_cast<const char*>(p.v) + head * EB;
    const char* dog = reinterpret_cast<const char*>(p.dout) + head * EB;

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
    const int kv_begin = (key_lo / BC) * BC;
    const int kv_end = CAUSAL ? min(key_hi, q0 + BR) : key_hi;
    const int n_tiles = kv_end > kv_begin ? (kv_end - kv_begin + BC - 1) / BC : 0;

    {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int off = tid * 16; off < 2 * TILEB; off += NT * 16) {
            *reinterpret_cast<FA_LDS u32x4*>((FA_LDS char*)buf0 + off) = z;
            *reinterpret_cast<FA_LDS u32x4*>((FA_LDS char*)buf1 + off) = z;
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

    // Q^T and dO^T as B operands: lane l holds query l%32, d = 16*dc + 8*(l/32) .. +7.
    u32x4 qop[NDC], doop[NDC];
    {
        const int qr = min(qw0 + col, N - 1);
        const char* qsrc = qg + (size_t)qr * ROWB + hh * 16;
        const char* dsrc = dog + (size_t)qr * ROWB + hh * 16;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
            qop[dc] = *reinterpret_cast<const u32x4*>(qsrc + dc * 32);
            doop[dc] = *reinterpret_cast<const u32x4*>(dsrc + dc * 32);
        }
    }
    const int qq = qw0 + col;
    float lse2 = INFINITY, dsum = 0.f;
    if (qq < N) {
        const float* grp = p.stats + ((size_t)bh * p.n_g + qq / 32) * 64;
        lse2 = grp[qq % 32];
        dsum = grp[32 + qq % 32];
    }

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    const float c = p.c;
    const bool wave_live = qw0 < N;

    const int sw_col = swz<CH>(col);
    const int tr_r = (lane & 15) >> 2;
    const int tr_c = lane & 3;
    const int tr_dsub = (lane >> 4) & 1;
    u32 v_off[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int row = 8 * half + 4 * hh + tr_r;
            const int chunk = 4 * db + 2 * tr_dsub + (tr_c >> 1);
            v_off[db][half] = (u32)(row * ROWB + ((chunk ^ swz<CH>(row)) << 4) + (tr_c & 1) * 8);
        }

    auto compute_tile = [&](int tile, const char* buf) {
        const int k0 = kv_begin + tile * BC;
        if (!wave_live || (CAUSAL && k0 > qw0 + 31)) return;
        const FA_LDS char* kt = (const FA_LDS char*)buf;
        const FA_LDS char* vt = (const FA_LDS char*)buf + TILEB;

        // ---- S^T = K_j Q^T and dP^T = V_j dO^T, one query per lane
        f32x16 s[NKB], dp[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = f32x16{};
            dp[kb] = f32x16{};
        }
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int off = (kb * 32 + col) * ROWB + (((2 * dc + hh) ^ sw_col) * 16);
                const u32x4 a = *reinterpret_cast<const FA_LDS u32x4*>(kt + off);
                s[kb] = mfma32x32x16<TI>(a, qop[dc], s[kb]);
                const u32x4 bv = *reinterpret_cast<const FA_LDS u32x4*>(vt + off);
                dp[kb] = mfma32x32x16<TI>(bv, doop[dc], dp[kb]);
            }
        }

        // ---- masks (as in the forward): register r of block kb is key
        // k0 + 4*hh + kb*32 + 8*(r/4) + r%4
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

        // ---- P^T = 2^(S^T c - lse2), dS^T = P^T (dP^T - D), packed as the B operand
        u32x4 pb[NKB][2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            float ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -lse2));
                ds[r] = pr * (dp[kb][r] - dsum);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) pb[kb][t][j] = pack2<TI>(ds[8 * t + 2 * j], ds[8 * t + 2 * j + 1]);
        }

        // ---- dQ^T += K_j^T dS^T (K^T by transpose reads of the K tile)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rowc = (kb * 32 + t * 16) * ROWB;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const i16x4 lo =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(kt + rowc + v_off[db][0]));
                    const i16x4 hi =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(kt + rowc + v_off[db][1]));
                    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
                    const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
                    const u32x4 a = {lo2[0], lo2[1], hi2[0], hi2[1]};
                    acc[db] = mfma32x32x16<TI>(a, pb[kb][t], acc[db]);
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

    if (qq < N) {
        char* row = reinterpret_cast<char*>(p.dq) + (head + (size_t)qq * D) * TO::kBytes;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * db + 8 * g + 4 * hh;
                const float v4[4] = {acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
                store_row4<TO>(row + d0 * TO::kBytes, v4, p.scale);
            }
    }
#endif
}

template <int D, int BC, int NW, typename TI, typename TO, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dq_kernel(BwdParams p) {
    bwd_dq_body<D, BC, NW, TI, TO, CAUSAL, MASK>(p, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------- dK, dV

template <int D, int BQ, int NW, typename TI, typename TO, bool CAUSAL, bool MASK>
__device__ __forceinline__ void bwd_dkdv_body(const BwdParams& p, int block, int grid) {
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BQ == 32 || BQ == 64, "query tile");
    static_assert(TI::kBytes == 2, "16-bit inputs");
    constexpr int NT = NW * 64;
    constexpr int BK = NW * 32;          // keys per workgroup
    constexpr int NQB = BQ / 32;
    constexpr int NDC = D / 16;
    constexpr int NDB = D / 32;
    constexpr int EB = 2;
    constexpr int ROWB = D * EB;
    constexpr int CH = ROWB / 16;
    constexpr int TILEB = BQ * ROWB;
    constexpr int RPI = 1024 / ROWB;
    constexpr int LOADS = TILEB / 1024;
    constexpr int LPW = (LOADS + NW - 1) / NW;
    constexpr int SB = NQB * 256;        // the tile's (lse2, D) groups

    // Two buffers, each Q, dO, then the stats groups; and the workgroup's K
    // rows, read as the B operand of S = Q K^T (in LDS rather than registers,
    // which leaves room for two waves per SIMD).
    __shared__ __attribute__((aligned(1024))) char buf0[2 * TILEB + SB];
    __shared__ __attribute__((aligned(1024))) char buf1[2 * TILEB + SB];
    __shared__ __attribute__((aligned(1024))) char kbuf[BK * ROWB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int hh = lane >> 5;

    // workgroup -> (batch*head, key tile); causal: the first key tiles see
    // the most queries, and they come first (work_item's order with the tile
    // index reversed).
    int split, bh, ktile;
    schedule(block, grid, p.n_ktiles, p.B * p.H, 1, p.head_group, p.xcd_remap, &split, &bh, &ktile);
    ktile = p.n_ktiles - 1 - ktile;
    const int b = bh / p.H;
    const int N = p.N;
    const int k0 = ktile * BK;
    const int kw0 = k0 + wave * 32;
    const int key = kw0 + col;

    const size_t head = (size_t)bh * (size_t)N * D;
    const char* qg = reinterpret_cast<const char*>(p.q) + head * EB;
    const char* kg = reinterpret_cast<const char*>(p.k) + head * EB;
    const char* vg = reinterpret_cast<const char*>(p.v) + head * EB;
    const char* dog = reinterpret_cast<const char*>(p.dout) + head * EB;
    const float* sg = p.stats + (size_t)bh * p.n_g * 64;

    bool kvalid = key < N;
    if constexpr (MASK) kvalid = kvalid && p.mask[(size_t)b * N + min(key, N - 1)] != 0;
    const bool all_valid = __builtin_amdgcn_ballot_w64(kvalid) == ~0ull;
    // Padded keys get dK = dV = 0 and contribute nothing: a wave whose 32
    // keys are all padded skips its products (it still takes part in the
    // tile barriers), and a workgroup with no valid key skips its loads and
    // the query loop and only stores its zeros.
    const bool wave_has_key = __builtin_amdgcn_ballot_w64(kvalid) != 0;
    const bool wg_has_key = !MASK || __syncthreads_or(wave_has_key ? 1 : 0) != 0;

    const int q_begin = CAUSAL ? (k0 / BQ) * BQ : 0;
    const int n_tiles = wg_has_key ? (N - q_begin + BQ - 1) / BQ : 0;

    {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int off = tid * 16; off < 2 * TILEB; off += NT * 16) {
            *reinterpret_cast<FA_LDS u32x4*>((FA_LDS char*)buf0 + off) = z;
            *reinterpret_cast<FA_LDS u32x4*>((FA_LDS char*)buf1 + off) = z;
        }
#pragma unroll
        for (int off = tid * 16; off < BK * ROWB; off += NT * 16)
            *reinterpret_cast<FA_LDS u32x4*>((FA_LDS char*)kbuf + off) = z;
        __syncthreads();
    }

    // The wave's 32 K rows into its own part of kbuf (row-major, chunks
    // swizzled as in the tiles); keys past N read as zero. Only this wave
    // reads them, so its own wait for the loads (the first tile's) suffices.
    if (n_tiles > 0) {
        constexpr int KLOADS = 32 * ROWB / 1024;  // wave loads per wave
        const int kbytes = max(N - kw0, 0) * ROWB;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)(kg + (size_t)min(kw0, N) * ROWB), 0, kbytes, kBufferFlags);
#pragma unroll
        for (int R = 0; R < KLOADS; ++R) {
            const int krow = R * RPI + lane / CH;
            const u32 off = (u32)(krow * ROWB + (((lane % CH) ^ swz<CH>(krow)) * 16));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FA_LDS void*)(kbuf + wave * 32 * ROWB + R * 1024), 16,
                                                     off, 0, 0, 0);
        }
    }

    u32 lane_off[LPW];
#pragma unroll
    for (int ii = 0; ii < LPW; ++ii) {
        const int R = wave + ii * NW;
        const int trow = R * RPI + lane / CH;
        lane_off[ii] = (u32)(trow * ROWB + (((lane % CH) ^ swz<CH>(trow)) * 16));
    }
    auto issue_tile = [&](int tile, char* buf) {
        const int q0 = q_begin + tile * BQ;
        const int bytes = (N - q0) * ROWB;  // rows past N read as 0
        const __amdgpu_buffer_rsrc_t rq =
            __builtin_amdgcn_make_buffer_rsrc((void*)(qg + (size_t)q0 * ROWB), 0, bytes, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rd =
            __builtin_amdgcn_make_buffer_rsrc((void*)(dog + (size_t)q0 * ROWB), 0, bytes, kBufferFlags);
#pragma unroll
        for (int ii = 0; ii < LPW; ++ii) {
            const int R = wave + ii * NW;
            if (LOADS % NW != 0 && R >= LOADS) break;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (FA_LDS void*)(buf + R * 1024), 16, lane_off[ii],
                                                     0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (FA_LDS void*)(buf + TILEB + R * 1024), 16,
                                                     lane_off[ii], 0, 0, 0);
        }
        // the tile's stats groups: 256 bytes each, one dword per lane; the
        // workspace is padded to a multiple of 64 queries, so they exist
        if (wave < NQB) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(sg + (size_t)(q0 / 32 + wave) * 64), 0, 256, kBufferFlags);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)(buf + 2 * TILEB + wave * 256), 4,
                                                     (u32)(lane * 4), 0, 0, 0);
        }
    };

    // V^T as a B operand held in registers: lane l holds key l%32, d = 16*dc +
    // 8*(l/32) .. +7. K^T, the same layout, is read from kbuf when needed.
    u32x4 vop[NDC];
    {
        const int kr = min(key, N - 1);
        const char* vsrc = vg + (size_t)kr * ROWB + hh * 16;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) vop[dc] = *reinterpret_cast<const u32x4*>(vsrc + dc * 32);
    }
    const FA_LDS char* kw = (const FA_LDS char*)kbuf + wave * 32 * ROWB + col * ROWB;

    f32x16 acc_dk[NDB], acc_dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        acc_dk[db] = f32x16{};
        acc_dv[db] = f32x16{};
    }
    const float c = p.c;
    const bool wave_live = kw0 < N;

    const int sw_col = swz<CH>(col);
    const int tr_r = (lane & 15) >> 2;
    const int tr_c = lane & 3;
    const int tr_dsub = (lane >> 4) & 1;
    u32 v_off[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int row = 8 * half + 4 * hh + tr_r;
            const int chunk = 4 * db + 2 * tr_dsub + (tr_c >> 1);
            v_off[db][half] = (u32)(row * ROWB + ((chunk ^ swz<CH>(row)) << 4) + (tr_c & 1) * 8);
        }

    auto compute_tile = [&](int tile, const char* buf) {
        if (!wave_live || !wave_has_key) return;
        const int q0 = q_begin + tile * BQ;
        const FA_LDS char* qt = (const FA_LDS char*)buf;
        const FA_LDS char* dt = (const FA_LDS char*)buf + TILEB;
        const FA_LDS char* st = (const FA_LDS char*)buf + 2 * TILEB;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            const int qblk0 = q0 + 32 * qb;
            // the whole block precedes the wave's keys, or lies past N
            if ((CAUSAL && qblk0 + 31 < kw0) || qblk0 >= N) continue;

            // ---- S = Q K^T and dP = dO V^T, one key per lane; register r
            // is query qblk0 + 8*(r/4) + 4*hh + r%4
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int dc = 0; dc < NDC; ++dc) {
                const int coff = ((2 * dc + hh) ^ sw_col) * 16;
                const int off = (qb * 32 + col) * ROWB + coff;
                const u32x4 a = *reinterpret_cast<const FA_LDS u32x4*>(qt + off);
                const u32x4 kb = *reinterpret_cast<const FA_LDS u32x4*>(kw + coff);
                s = mfma32x32x16<TI>(a, kb, s);
                const u32x4 g = *reinterpret_cast<const FA_LDS u32x4*>(dt + off);
                dp = mfma32x32x16<TI>(g, vop[dc], dp);
            }
            // ---- masks: invalid key (this lane's column), causal q < key.
            // Queries past N carry lse2 = +inf and need no test.
            const bool diag = CAUSAL && (qblk0 < kw0 + 31);
            if (!all_valid || diag) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qi = qblk0 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    const bool ok = kvalid && (!CAUSAL || qi >= key);
                    s[r] = ok ? s[r] : -INFINITY;
                }
            }
            // ---- P = 2^(S c - lse2), dS = P (dP - D), both packed as B
            // operands; registers 4g..4g+3 are queries 8g + 4*hh .. +3, whose
            // (lse2, D) are read from the stats group one f32x4 each
            u32x4 pb[2], sb[2];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 lv = *reinterpret_cast<const FA_LDS f32x4*>(st + qb * 256 + (8 * g + 4 * hh) * 4);
                const f32x4 dv4 =
                    *reinterpret_cast<const FA_LDS f32x4*>(st + qb * 256 + 128 + (8 * g + 4 * hh) * 4);
                float pr[4], ds[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + i], c, -lv[i]));
                    ds[i] = pr[i] * (dp[4 * g + i] - dv4[i]);
                }
                const int t = g >> 1, j = 2 * (g & 1);
                pb[t][j] = pack2<TI>(pr[0], pr[1]);
                pb[t][j + 1] = pack2<TI>(pr[2], pr[3]);
                sb[t][j] = pack2<TI>(ds[0], ds[1]);
                sb[t][j + 1] = pack2<TI>(ds[2], ds[3]);
            }
            // ---- dV^T += dO^T P and dK^T += Q^T dS (transpose reads of the dO and Q tiles)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rowc = (qb * 32 + t * 16) * ROWB;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const i16x4 glo =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(dt + rowc + v_off[db][0]));
                    const i16x4 ghi =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(dt + rowc + v_off[db][1]));
                    const u32x2 glo2 = __builtin_bit_cast(u32x2, glo);
                    const u32x2 ghi2 = __builtin_bit_cast(u32x2, ghi);
                    const u32x4 ga = {glo2[0], glo2[1], ghi2[0], ghi2[1]};
                    acc_dv[db] = mfma32x32x16<TI>(ga, pb[t], acc_dv[db]);
                    const i16x4 qlo =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(qt + rowc + v_off[db][0]));
                    const i16x4 qhi =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(qt + rowc + v_off[db][1]));
                    const u32x2 qlo2 = __builtin_bit_cast(u32x2, qlo);
                    const u32x2 qhi2 = __builtin_bit_cast(u32x2, qhi);
                    const u32x4 qa = {qlo2[0], qlo2[1], qhi2[0], qhi2[1]};
                    acc_dk[db] = mfma32x32x16<TI>(qa, sb[t], acc_dk[db]);
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

    if (key < N) {
        char* krow = reinterpret_cast<char*>(p.dk) + (head + (size_t)key * D) * TO::kBytes;
        char* vrow = reinterpret_cast<char*>(p.dv) + (head + (size_t)key * D) * TO::kBytes;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * db + 8 * g + 4 * hh;
                const float k4[4] = {acc_dk[db][4 * g], acc_dk[db][4 * g + 1], acc_dk[db][4 * g + 2],
                                     acc_dk[db][4 * g + 3]};
                const float v4[4] = {acc_dv[db][4 * g], acc_dv[db][4 * g + 1], acc_dv[db][4 * g + 2],
                                     acc_dv[db][4 * g + 3]};
                store_row4<TO>(krow + d0 * TO::kBytes, k4, p.scale);
                store_row4<TO>(vrow + d0 * TO::kBytes, v4, 1.f);
            }
    }
#endif
}

// At least two waves per SIMD: with K in LDS the kernel fits 256 registers.
template <int D, int BQ, int NW, typename TI, typename TO, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void attn_bwd_dkdv_kernel(
    BwdParams p) {
    bwd_dkdv_body<D, BQ, NW, TI, TO, CAUSAL, MASK>(p, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------- dK, dV and dQ in one launch

// Workgroups [0, n_dkdv_blocks) run the dK/dV body, the rest the dQ body;
// the two are independent once the prep kernel has run. With both in one
// grid the hardware starts dQ workgroups in the slots that the last round of
// dK/dV workgroups leaves idle, instead of the dK/dV kernel ending on a
// partly empty round and the dQ kernel on another. Used at d = 64, where the
// two bodies' LDS together (about 50 KB) still leave three workgroups per CU;
// at d = 128 it would leave one.
template <int D, int BC, int BQ, int NW, typename TI, typename TO, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(NW * 64) void attn_bwd_fused_kernel(BwdParams p) {
    const int nk = p.n_dkdv_blocks;
    if ((int)blockIdx.x < nk) bwd_dkdv_body<D, BQ, NW, TI, TO, CAUSAL, MASK>(p, (int)blockIdx.x, nk);
    else bwd_dq_body<D, BC, NW, TI, TO, CAUSAL, MASK>(p, (int)blockIdx.x - nk, (int)gridDim.x - nk);
}

}  // namespace fa
