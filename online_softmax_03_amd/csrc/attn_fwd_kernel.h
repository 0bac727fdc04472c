// Attention forward with online softmax for gfx950 (MI355X): the kernel template.
//
// One workgroup owns B_r = 32*NW query rows of one (batch, head); each of its
// NW waves owns 32 of them. The workgroup walks the key/value sequence in
// tiles of B_c rows ("Online Softmax 算法详解" section 2.3: only K/V blocks are
// looped over; every query row keeps its own state, "在线Softmax算法解析"
// section 3.3). Per tile:
//
//   1. K_j and V_j land in LDS straight from HBM (global_load_lds_dwordx4,
//      16 bytes per lane, coalesced), double-buffered so the next tile's load
//      overlaps this tile's math.
//   2. S^T = K_j * Q^T on v_mfma_f32_32x32x16 (bf16/fp16 in, fp32 out). The
//      transposed product puts one query per lane column: lane l holds query
//      l%32 and 16 of the tile's 32 keys per 32-key block, the other 16 sit in
//      lane l^32. Row max and row sum are then in-lane reductions plus a single
//      v_permlane32_swap, instead of a 32-lane butterfly.
//   3. Mask (causal diagonal, key padding, sequence tail) by writing -inf.
//   4. Online update in raw score units with the scale folded into exp2
//      ("Online Softmax 算法详解" sections 4.3, 4.5, 5): m_new = max(m, rowmax),
//      alpha = 2^((m - m_new)*c), l = alpha*l + sum P, P = 2^(s*c - m_new*c)
//      as one FMA plus v_exp_f32, c = scale*log2(e). The -inf guard of section
//      7.1 uses 0 as the subtrahend when m_new is still -inf. O is rescaled
//      only when some row maximum in the wave actually moved (the conditional
//      rescale of "在线Softmax算法解析" section 2.1, step 3).
//   5. P is rounded to bf16/fp16 in registers and fed straight back as the B
//      operand of O^T += V_j^T * P^T: the MFMA result layout of S^T matches the
//      operand layout up to a fixed permutation of keys inside each 16-key
//      group, and the V^T operand is read from the row-major V tile with
//      ds_read_b64_tr_b16 in that same key order. No LDS round trip for P.
//
// After the last tile: the two lane halves' row sums are added (the deferred
// cross-lane reduce of "Online Softmax 算法详解" section 4.6), inv = 1/l with the
// l == 0 / NaN guard of section 7.2, O *= inv, LSE = (m*c + log2 l)*ln 2 with
// the -inf case of section 7.3, and O and LSE are stored.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef unsigned int u32;
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define FA_LDS __attribute__((address_space(3)))
#define FA_GLOBAL __attribute__((address_space(1)))

// Element tags.
struct BF16 { static constexpr int kBytes = 2; };
struct F16 { static constexpr int kBytes = 2; };
struct F32 { static constexpr int kBytes = 4; };

struct Params {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const uint8_t* mask;  // [B][N] or nullptr
    int B, H, N;
    int n_qtiles;         // ceil(N / B_r)
    int xcd_remap;        // 1: group consecutive tiles of a head on one XCD
    float c;              // scale * log2(e)
};

constexpr float kLn2 = 0.69314718055994530942f;

// ---------------------------------------------------------------- helpers

template <typename T>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mfma32x32x16<BF16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mfma32x32x16<F16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two floats rounded to nearest-even into one packed 32-bit register.
template <typename T>
__device__ __forceinline__ u32 pack2(float lo, float hi);

template <>
__device__ __forceinline__ u32 pack2<BF16>(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(u32, r);
}

template <>
__device__ __forceinline__ u32 pack2<F16>(float lo, float hi) {
    f16x2 r = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(u32, r);
}

// Value of x combined with the value in lane l^32 (one v_permlane32_swap).
// After swap(x, x) the lower half holds (own, upper partner) and the upper
// half (lower partner, own), so both halves combine the pair in the same order.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS tile layout: row-major [B_c][D] with the 16-byte chunk index XORed by a
// row-dependent pattern, so that the K operand reads (16 rows x one chunk per
// 16 lanes) and the V transpose reads (4 rows x 4 chunks per 16 lanes) hit
// distinct bank groups.
template <int D>
__device__ __forceinline__ constexpr int swz(int row) {
    if constexpr (D == 128) {
        return ((row & 3) << 2) | ((row >> 2) & 3);
    } else {
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    }
}

__device__ __forceinline__ void wait_vmcnt0() {
    // s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their no-wait maxima.
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <typename T>
__device__ __forceinline__ void store_row4(char* dst, const float* v4, float inv);

template <>
__device__ __forceinline__ void store_row4<F32>(char* dst, const float* v4, float inv) {
    f32x4 r = {v4[0] * inv, v4[1] * inv, v4[2] * inv, v4[3] * inv};
    *reinterpret_cast<f32x4*>(dst) = r;
}

template <>
__device__ __forceinline__ void store_row4<BF16>(char* dst, const float* v4, float inv) {
    u32x2 r = {pack2<BF16>(v4[0] * inv, v4[1] * inv), pack2<BF16>(v4[2] * inv, v4[3] * inv)};
    *reinterpret_cast<u32x2*>(dst) = r;
}

template <>
__device__ __forceinline__ void store_row4<F16>(char* dst, const float* v4, float inv) {
    u32x2 r = {pack2<F16>(v4[0] * inv, v4[1] * inv), pack2<F16>(v4[2] * inv, v4[3] * inv)};
    *reinterpret_cast<u32x2*>(dst) = r;
}

// First and last index j in [0, n) with row[j] != 0, over the whole
// workgroup. Returns {INT32_MAX, -1} when there is none.
template <int NT>
__device__ __forceinline__ void mask_extent(const uint8_t* row, int n, int* first, int* last) {
    __shared__ int s_first[NT / 64], s_last[NT / 64];
    int f = 0x7fffffff, l = -1;
    for (int j = threadIdx.x; j < n; j += NT) {
        if (row[j] != 0) {
            f = min(f, j);
            l = max(l, j);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        f = min(f, __shfl_xor(f, off));
        l = max(l, __shfl_xor(l, off));
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_first[w] = f;
        s_last[w] = l;
    }
    __syncthreads();
    f = s_first[0];
    l = s_last[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) {
        f = min(f, s_first[i]);
        l = max(l, s_last[i]);
    }
    *first = f;
    *last = l;
}

// ---------------------------------------------------------------- kernel

template <int D, int BC, int NW, typename TI, typename TO, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(Params p) {
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BC % 32 == 0 && BC >= 32 && BC <= 128, "key tile");
    static_assert(TI::kBytes == 2, "16-bit inputs on this path");
    constexpr int NT = NW * 64;
    constexpr int BR = NW * 32;          // query rows per workgroup
    constexpr int NKB = BC / 32;         // 32-key blocks per tile
    constexpr int NDC = D / 16;          // 16-wide slices of d (QK contraction steps)
    constexpr int NDB = D / 32;          // 32-wide blocks of d in O^T
    constexpr int CH = D / 8;            // 16-byte chunks per row
    constexpr int ROWB = D * 2;          // bytes per row
    constexpr int TILEB = BC * ROWB;     // bytes per K or V tile
    constexpr int RPI = 1024 / ROWB;     // tile rows per 1 KB wave load
    constexpr int LOADS = TILEB / 1024;  // wave loads per tensor per tile
    constexpr int LPW = (LOADS + NW - 1) / NW;

    __shared__ __attribute__((aligned(1024))) char smem[2][2][TILEB];  // [buffer][K, V]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;  // query within the wave's 32
    const int hh = lane >> 5;   // which 16 of every 32 keys this lane holds

    // workgroup -> (batch*head, query tile). Query tiles of one head are walked
    // from the last (largest causal extent) to the first, and with the remap
    // consecutive ids of one XCD (ids are dealt round-robin over 8 XCDs) cover
    // consecutive tiles, so the workgroups sharing a head's K/V share an L2.
    int id = blockIdx.x;
    if (p.xcd_remap) id = (id & 7) * (gridDim.x >> 3) + (id >> 3);
    const int bh = id / p.n_qtiles;
    const int qt = p.n_qtiles - 1 - (id - bh * p.n_qtiles);
    const int b = bh / p.H;
    const int N = p.N;
    const int q0 = qt * BR;
    const int qw0 = q0 + wave * 32;

    const size_t head = (size_t)bh * (size_t)N * D;
    const char* qg = reinterpret_cast<const char*>(p.q) + head * 2;
    const char* kg = reinterpret_cast<const char*>(p.k) + head * 2;
    const char* vg = reinterpret_cast<const char*>(p.v) + head * 2;

    // Key range this workgroup must visit.
    int kv_begin = 0;
    int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const uint8_t* mrow = MASK ? p.mask + (size_t)b * N : nullptr;
    if constexpr (MASK) {
        int first, last;
        mask_extent<NT>(mrow, kv_end, &first, &last);
        if (last < 0) {
            kv_end = 0;
        } else {
            kv_begin = (first / BC) * BC;
            kv_end = last + 1;
        }
    }
    const int n_tiles = kv_end > kv_begin ? (kv_end - kv_begin + BC - 1) / BC : 0;

    // Issue one tile's K and V loads into LDS buffer `buf`. Wave load R fills
    // bytes [R*1024, R*1024+1024) of the tile: lane s writes slot s of that
    // range, i.e. row R*RPI + s/CH, physical chunk s%CH, which holds logical
    // chunk (s%CH) ^ swz(row). Rows past N read row N-1 (finite data; those
    // keys are masked).
    auto issue_tile = [&](int tile, int buf) {
        const int k0 = kv_begin + tile * BC;
#pragma unroll
        for (int ii = 0; ii < LPW; ++ii) {
            const int R = wave + ii * NW;
            if (LOADS % NW != 0 && R >= LOADS) break;
            const int trow = R * RPI + lane / CH;
            const int row = min(k0 + trow, N - 1);
            const int chunk = (lane % CH) ^ swz<D>(trow);
            const size_t off = (size_t)row * ROWB + chunk * 16;
            __builtin_amdgcn_global_load_lds((const FA_GLOBAL void*)(kg + off),
                                             (FA_LDS void*)(&smem[buf][0][R * 1024]), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const FA_GLOBAL void*)(vg + off),
                                             (FA_LDS void*)(&smem[buf][1][R * 1024]), 16, 0, 0);
        }
    };

    // Q^T as the B operand: lane l holds query l%32, d = 16*dc + 8*(l/32) .. +7.
    u32x4 qop[NDC];
    {
        const int qr = min(qw0 + col, N - 1);
        const char* src = qg + (size_t)qr * ROWB + hh * 16;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) qop[dc] = *reinterpret_cast<const u32x4*>(src + dc * 32);
    }

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    float m_run = -INFINITY;  // running row max, raw q.k units
    float l_run = 0.f;        // this lane's share of the running row sum
    const float c = p.c;
    const bool wave_live = qw0 < N;

    // Per-lane geometry of the V^T transpose reads (see the PV step).
    const int g16 = lane >> 4;
    const int tr_r = (lane & 15) >> 2;   // which of 4 consecutive keys this lane addresses
    const int tr_c = lane & 3;           // which 4-wide d slice it addresses
    const int tr_dsub = g16 & 1;         // which 16 of the 32 d values the group covers
    const int sw_k = swz<D>(col) ^ hh;   // K operand: chunk (2*dc + hh) ^ swz(row)

    if (n_tiles > 0) issue_tile(0, 0);

    for (int it = 0; it < n_tiles; ++it) {
        const int buf = it & 1;
        const int k0 = kv_begin + it * BC;
        wait_vmcnt0();     // this wave's loads of tile `it` have landed
        __syncthreads();   // ... everyone's, and tile it-1 is no longer read
        if (it + 1 < n_tiles) issue_tile(it + 1, buf ^ 1);

        // Waves whose queries all precede this tile's first key have nothing to do.
        const bool need = wave_live && (!CAUSAL || k0 <= qw0 + 31);
        if (!need) continue;

        const char* kt = &smem[buf][0][0];
        const char* vt = &smem[buf][1][0];

        // ---- S^T = K_j Q^T
        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int row = kb * 32 + col;
                const int chunk = (2 * dc) ^ sw_k;
                const u32x4 a = *reinterpret_cast<const FA_LDS u32x4*>(
                    (const FA_LDS char*)kt + row * ROWB + chunk * 16);
                s[kb] = mfma32x32x16<TI>(a, qop[dc], s[kb]);
            }
        }

        // ---- masks: keys past the range, the causal diagonal, padded keys
        const bool diag = CAUSAL && (k0 + BC - 1 > qw0);
        const bool tail = k0 + BC > kv_end;
        if (MASK || diag || tail) {
            const int qq = qw0 + col;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    bool ok = key < kv_end;
                    if (CAUSAL) ok = ok && key <= qq;
                    if (MASK) ok = ok && mrow[min(key, N - 1)] != 0;
                    s[kb][r] = ok ? s[kb][r] : -INFINITY;
                }
            }
        }

        // ---- online softmax update
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = pair_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float ref = (m_new == -INFINITY) ? 0.f : m_new * c;
        const float alpha = __builtin_amdgcn_exp2f(m_run * c - ref);
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -ref));
                s[kb][r] = e;
                rs += e;
            }
        l_run = l_run * alpha + rs;
        m_run = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
        }

        // ---- P^T as the B operand: 16-key group t of block kb is registers 8t..8t+7
        u32x4 pb[NKB][2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    pb[kb][t][j] = pack2<TI>(s[kb][8 * t + 2 * j], s[kb][8 * t + 2 * j + 1]);

        // ---- O^T += V_j^T P^T. Register j of the B operand above is key
        // 16t + 8(j/4) + 4*hh + j%4 of the block; the A operand must hold
        // V[that key][d = l%32] in the same slot. Two ds_read_b64_tr_b16 give
        // it: within each 16-lane group, lane 4r+c addresses V[key0 + r][dbase
        // + 4c .. +3], and after the transpose lane i holds V[key0 .. key0+3]
        // [dbase + i].
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int row0 = kb * 32 + t * 16 + 4 * hh + tr_r;
                const int row1 = row0 + 8;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int chunk = 4 * db + 2 * tr_dsub + (tr_c >> 1);
                    const int within = (tr_c & 1) * 8;
                    const FA_LDS char* a0 = (const FA_LDS char*)vt + row0 * ROWB +
                                            ((chunk ^ swz<D>(row0)) << 4) + within;
                    const FA_LDS char* a1 = (const FA_LDS char*)vt + row1 * ROWB +
                                            ((chunk ^ swz<D>(row1)) << 4) + within;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)a0);
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)a1);
                    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
                    const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
                    const u32x4 a = {lo2[0], lo2[1], hi2[0], hi2[1]};
                    acc[db] = mfma32x32x16<TI>(a, pb[kb][t], acc[db]);
                }
            }
        }
    }

    // ---- finalize and store
    const float l_tot = pair_sum(l_run);
    const bool dead = !(l_tot > 0.f);  // no allowed key (sum 0) or NaN
    const float inv = dead ? 0.f : 1.f / l_tot;
    const float lse = dead ? -INFINITY : (m_run * c + __builtin_amdgcn_logf(l_tot)) * kLn2;
    const int qq = qw0 + col;
    if (qq < N) {
        char* orow = reinterpret_cast<char*>(p.o) + (head + (size_t)qq * D) * TO::kBytes;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * db + 8 * g + 4 * hh;
                const float v4[4] = {acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2],
                                     acc[db][4 * g + 3]};
                store_row4<TO>(orow + d0 * TO::kBytes, v4, inv);
            }
        if (hh == 0) p.lse[(size_t)bh * N + qq] = lse;
    }
}

}  // namespace fa
