// Attention forward with online softmax for gfx950 (MI355X): types and device
// helpers shared by the 16-bit kernel (attn_fwd_kernel.h) and the fp32 kernel
// (attn_fwd_f32_kernel.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "work_item.h"

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
    int xcd_remap;        // XcdMode: how workgroup ids spread over the 8 XCDs
    int head_group;       // heads whose query tiles are dealt together (>= 1)
    int fair;             // 1: equal-progress wave priorities (see fa_api.hip)
    float c;              // scale * log2(e)
    // split-KV only: the key tiles of every query tile are cut into n_splits
    // contiguous parts (with split_u > 0, under a causal mask: parts_of(...)
    // <= n_splits parts of at most split_u * B_r / B_c key tiles each,
    // work_item.h, split_parts = parts_per_head workgroups per head); part s
    // writes its normalised partial output and its LSE to ws_o
    // [n_splits][B*H][N][d] and ws_lse [n_splits][B*H][N].
    int n_splits;
    int split_u;
    long long split_parts;
    float* ws_o;
    float* ws_lse;
};

// Workgroup -> (key-range part `split` of `n_parts`, batch*head `bh`, query
// tile `qt`) for the attention kernels (work_item.h).
template <bool SPLIT, bool CAUSAL>
__device__ __forceinline__ void attn_schedule(const Params& p, int* split, int* n_parts, int* bh, int* qt) {
    if constexpr (SPLIT && CAUSAL) {
        if (p.split_u > 0) {
            long long k = 0;
            schedule_parts((int)blockIdx.x, (int)gridDim.x, p.split_parts, p.xcd_remap, bh, &k);
            locate_part(k, p.n_qtiles, p.split_u, p.n_splits, qt, split);
            *n_parts = parts_of(*qt, p.n_qtiles, p.split_u, p.n_splits);
            return;
        }
    }
    *n_parts = SPLIT ? p.n_splits : 1;
    schedule((int)blockIdx.x, (int)gridDim.x, p.n_qtiles, p.B * p.H, *n_parts, p.head_group, p.xcd_remap, split,
             bh, qt);
}

constexpr float kLn2 = 0.69314718055994530942f;
// Largest growth of a row maximum, in log2 units of the exponent, tolerated
// before the state is rescaled: P stays below 2^8 = 256.
constexpr float kRescaleLog2 = 8.0f;
// Word 3 of a raw buffer resource on gfx9: 32-bit data format, no swizzle.
constexpr int kBufferFlags = 0x00020000;

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

// fp32 inputs: one k-pair per instruction. A: lane l holds A[l%32][l/32];
// B: lane l holds B[l/32][l%32]; the result layout is that of the 16-bit forms.
__device__ __forceinline__ f32x16 mfma32x32x2_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
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

// LDS tile layout: row-major [B_c][row bytes] with the 16-byte chunk index
// XORed by a row-dependent pattern, so that the K operand reads (16 rows x one
// chunk per 16 lanes) and the V transpose reads (4 rows x 4 chunks per 16
// lanes) hit distinct bank groups.
//   CH = 8 chunks per row (bf16/fp16, d = 64):  ((row>>1)&1)<<2 | (row>>2)&3
//   CH >= 16 (bf16/fp16 d = 128, fp32):        (row&3)<<2 | (row>>2)&3
template <int CH>
__device__ __forceinline__ constexpr int swz(int row) {
    if constexpr (CH >= 16) {
        return ((row & 3) << 2) | ((row >> 2) & 3);
    } else {
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    }
}

__device__ __forceinline__ void wait_vmcnt0() {
    // s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their no-wait maxima.
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

__device__ __forceinline__ void wait_lgkmcnt0() {
    // s_waitcnt lgkmcnt(0); vmcnt (both fields) and expcnt left at their
    // no-wait maxima.
    __builtin_amdgcn_s_waitcnt(0xC07F);
}

// Four consecutive values of an output row, times `inv`, in the output type
// (16 bytes for fp32, 8 for bf16/fp16, rounded to nearest even). Plain
// stores: the non-temporal hint (`nt`) on these per-lane pieces of 32 rows
// was measured at 4.4x the algorithmic HBM write bytes on the headline
// workload (575 against 130 MiB per launch; 1.7x for fp32 O at d = 64),
// where the L2 otherwise merges them into whole lines.
template <typename T>
__device__ __forceinline__ void store_row4(char* dst, const float* v4, float inv) {
    if constexpr (std::is_same_v<T, F32>) {
        const f32x4 r = {v4[0] * inv, v4[1] * inv, v4[2] * inv, v4[3] * inv};
        *reinterpret_cast<f32x4*>(dst) = r;
    } else {
        const u32x2 r = {pack2<T>(v4[0] * inv, v4[1] * inv), pack2<T>(v4[2] * inv, v4[3] * inv)};
        *reinterpret_cast<u32x2*>(dst) = r;
    }
}

// Valid-key extent of one mask row over [0, n): the first and last index
// with row[j] != 0 and the number of such indices, reduced over the whole
// workgroup. first = INT32_MAX, last = -1 when there is none.
template <int NT>
__device__ __forceinline__ void mask_extent(const uint8_t* row, int n, int* first, int* last,
                                            int* count) {
    __shared__ int s_red[3][NT / 64];
    int f = 0x7fffffff, l = -1, cnt = 0;
    for (int j = threadIdx.x; j < n; j += NT) {
        if (row[j] != 0) {
            f = min(f, j);
            l = max(l, j);
            ++cnt;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        f = min(f, __shfl_xor(f, off));
        l = max(l, __shfl_xor(l, off));
        cnt += __shfl_xor(cnt, off);
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_red[0][w] = f;
        s_red[1][w] = l;
        s_red[2][w] = cnt;
    }
    __syncthreads();
    f = s_red[0][0];
    l = s_red[1][0];
    cnt = s_red[2][0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) {
        f = min(f, s_red[0][i]);
        l = max(l, s_red[1][i]);
        cnt += s_red[2][i];
    }
    *first = f;
    *last = l;
    *count = cnt;
}

}  // namespace fa
