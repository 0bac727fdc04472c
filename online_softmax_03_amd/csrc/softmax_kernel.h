// Row softmax with the online normaliser on gfx950 (MI355X).
//
// For every row x of a [rows][cols] matrix: y = exp(x - m) / l with
// m = max x and l = sum exp(x - m), plus LSE = m + ln l. The method is the
// two-pass online softmax of "Online Softmax 算法详解" section 2.2: the first
// pass produces m and l together by the incremental update (a new maximum
// rescales the running sum by exp(m_old - m_new)), the second pass writes
// the normalised values. Partial (m, l) states of different parts of a row
// combine with the merge of the online-softmax interview card (section 三):
// m = max(m1, m2), l = l1 e^(m1 - m) + l2 e^(m2 - m). exp is evaluated as
// exp2 of (x - m) * log2(e); the subtraction comes first so that large inputs
// close to the maximum keep their precision. Entries equal to -inf are
// masked; a row with no finite entry gets y = 0 and LSE = -inf exactly (the
// guards of "Online Softmax 算法详解" sections 7.1-7.3).
//
// Two kernels, both HBM-bound:
//   softmax_resident_kernel: the row stays in registers, so x is read from
//     HBM once and y written once. Each thread takes a slice of the row
//     (16-byte vectors, coalesced across the threads of the row), computes
//     the slice's maximum and the sum of its exponentials (kept in
//     registers), the slices' (m, l) states are merged across the lanes of a
//     wave (butterfly, bitwise identical in every lane because the merge is
//     commutative in IEEE arithmetic) and across the waves of the row (LDS,
//     in a fixed order), and each thread rescales its exponentials by
//     e^(m_slice - m) / l.
//   softmax_resident_lds_kernel: rows longer than the registers of one
//     workgroup hold: each thread keeps part of its slice in registers and
//     the rest in LDS (loaded there by LDS DMA, no registers in between), so
//     x is still read from HBM once. One workgroup per compute unit walks
//     several rows and loads the next row while it writes the current one.
//   softmax_stream_kernel: rows too long for registers and LDS, or whose
//     length is not a whole number of 16-byte vectors. Pass 1 streams the row and keeps
//     a running (m, l) per thread, updated per vector; pass 2 streams it again
//     and writes y. One workgroup per row.
#pragma once

#include "attn_common.h"
#include "softmax_table.h"

namespace fa {

constexpr float kSmLog2e = 1.44269504088896340736f;

// ---------------------------------------------------------------- element I/O

// One 16-byte input vector as floats: 8 (bf16, fp16) or 4 (fp32) values.
template <typename T>
struct VecIn;

template <>
struct VecIn<BF16> {
    static constexpr int kN = 8;
    __device__ static void load(const char* p, float* v) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(u[i] << 16);
            v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    __device__ static float load1(const char* p) {
        return __uint_as_float((u32)(*reinterpret_cast<const unsigned short*>(p)) << 16);
    }
    __device__ static void cvt(const u32x4& u, float* v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(u[i] << 16);
            v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    __device__ static void load_lds(const FA_LDS char* p, float* v) {
        const u32x4 u = *reinterpret_cast<const FA_LDS u32x4*>(p);
        cvt(u, v);
    }
};

template <>
struct VecIn<F16> {
    static constexpr int kN = 8;
    __device__ static void load(const char* p, float* v) {
        const f16x8 h = *reinterpret_cast<const f16x8*>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
    }
    __device__ static float load1(const char* p) { return (float)*reinterpret_cast<const _Float16*>(p); }
    __device__ static void cvt(const u32x4& u, float* v) {
        const f16x8 h = __builtin_bit_cast(f16x8, u);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
    }
    __device__ static void load_lds(const FA_LDS char* p, float* v) {
        const u32x4 u = *reinterpret_cast<const FA_LDS u32x4*>(p);
        cvt(u, v);
    }
};

template <>
struct VecIn<F32> {
    static constexpr int kN = 4;
    __device__ static void load(const char* p, float* v) {
        const f32x4 f = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = f[i];
    }
    __device__ static float load1(const char* p) { return *reinterpret_cast<const float*>(p); }
    __device__ static void cvt(const u32x4& u, float* v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(u[i]);
    }
    __device__ static void load_lds(const FA_LDS char* p, float* v) {
        const u32x4 u = *reinterpret_cast<const FA_LDS u32x4*>(p);
        cvt(u, v);
    }
};

// N values times s, rounded to the output dtype and stored at p (N * size
// bytes, 16-byte aligned when N * size is a multiple of 16).
template <typename T, int N>
__device__ __forceinline__ void store_scaled(char* p, const float* v, float s) {
    if constexpr (T::kBytes == 4) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const f32x4 r = {v[i] * s, v[i + 1] * s, v[i + 2] * s, v[i + 3] * s};
            *reinterpret_cast<f32x4*>(p + 4 * i) = r;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 8) {
            const u32x4 r = {pack2<T>(v[i] * s, v[i + 1] * s), pack2<T>(v[i + 2] * s, v[i + 3] * s),
                             pack2<T>(v[i + 4] * s, v[i + 5] * s), pack2<T>(v[i + 6] * s, v[i + 7] * s)};
            *reinterpret_cast<u32x4*>(p + 2 * i) = r;
        }
    }
}

// As store_scaled, through a buffer resource at per-lane byte offset
// voffset (stores outside the resource are dropped by the hardware).
template <typename T, int N>
__device__ __forceinline__ void store_scaled_buf(__amdgpu_buffer_rsrc_t r, u32 voffset, const float* v, float s) {
    if constexpr (T::kBytes == 4) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const u32x4 q = {__float_as_uint(v[i] * s), __float_as_uint(v[i + 1] * s),
                             __float_as_uint(v[i + 2] * s), __float_as_uint(v[i + 3] * s)};
            __builtin_amdgcn_raw_buffer_store_b128(q, r, voffset + 4 * i, 0, 0);
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 8) {
            const u32x4 q = {pack2<T>(v[i] * s, v[i + 1] * s), pack2<T>(v[i + 2] * s, v[i + 3] * s),
                             pack2<T>(v[i + 4] * s, v[i + 5] * s), pack2<T>(v[i + 6] * s, v[i + 7] * s)};
            __builtin_amdgcn_raw_buffer_store_b128(q, r, voffset + 2 * i, 0, 0);
        }
    }
}

template <typename T>
__device__ __forceinline__ void store1(char* p, float v) {
    if constexpr (T::kBytes == 4) {
        *reinterpret_cast<float*>(p) = v;
    } else {
        const u32 w = pack2<T>(v, 0.f);
        *reinterpret_cast<unsigned short*>(p) = (unsigned short)(w & 0xffffu);
    }
}

// ---------------------------------------------------------------- (m, l) states

// exp2 of the exponent offset that brings a state with maximum `m` to the
// reference `ref` (log2(e) folded in); 0 for an empty state.
__device__ __forceinline__ float sm_rescale(float m, float ref) {
    return __builtin_amdgcn_exp2f((m - ref) * kSmLog2e);
}

// Merge of two partial states (m1, l1) and (m2, l2), in place into (m, l).
// Symmetric in its two arguments, so every lane of a butterfly ends with the
// same bits: the two products are rounded separately (no contraction into a
// fused multiply-add, which would round them differently depending on the
// argument order) before the commutative add.
__device__ __forceinline__ void sm_merge(float& m, float& l, float m2, float l2) {
#pragma clang fp contract(off)
    const float mm = fmaxf(m, m2);
    const float ref = (mm == -INFINITY) ? 0.f : mm;
    l = l * sm_rescale(m, ref) + l2 * sm_rescale(m2, ref);
    m = mm;
}

// The value of lane l ^ K (K < 32) by ds_swizzle in its bit-mask mode (and
// mask 0x1f, xor mask K, within each 32-lane half): no lane index needed.
template <int K>
__device__ __forceinline__ float lane_xor(float x) {
    static_assert(K >= 1 && K <= 16, "xor within 32 lanes");
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (K << 10) | 0x1f));
}

template <int K>
__device__ __forceinline__ void sm_xor_merge(float& m, float& l) {
    if constexpr (K >= 1) {
        sm_merge(m, l, lane_xor<K>(m), lane_xor<K>(l));
        sm_xor_merge<K / 2>(m, l);
    }
}

// Merge over the 64 lanes of a wave; every lane ends with the wave's state.
// The two 32-lane halves first, by v_permlane32_swap, which hands every lane
// the states of lanes l % 32 and 32 + l % 32 in that order; then xor steps
// of 16 ... 1 within each half.
__device__ __forceinline__ void sm_wave_merge(float& m, float& l) {
    const auto ms = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    const auto ls = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    m = __uint_as_float(ms[0]);
    l = __uint_as_float(ls[0]);
    sm_merge(m, l, __uint_as_float(ms[1]), __uint_as_float(ls[1]));
    sm_xor_merge<16>(m, l);
}

// ---------------------------------------------------------------- resident rows

// WPR waves per row, RPB rows per workgroup, VPT 16-byte input vectors per
// thread: rows of up to WPR * 64 * VPT vectors. cols must be a multiple of
// the vector width; rows start 16-byte aligned.
template <typename TI, typename TO, int WPR, int RPB, int VPT>
__global__ __launch_bounds__(WPR * RPB * 64) void softmax_resident_kernel(SoftmaxParams sp) {
    constexpr int E = VecIn<TI>::kN;
    constexpr int RT = WPR * 64;  // threads per row
    __shared__ float s_m[RPB][WPR], s_l[RPB][WPR];

    const int tid = threadIdx.x;
    const int grp = tid / RT;       // row slot within the workgroup
    const int t = tid % RT;         // thread within the row
    const int wave_in_row = t >> 6;
    const long long row = (long long)blockIdx.x * RPB + grp;
    const bool live = row < sp.rows;
    const int nvec = sp.cols / E;

    const char* xr = reinterpret_cast<const char*>(sp.x) + (live ? row : 0) * (long long)sp.cols * TI::kBytes;
    char* yr = reinterpret_cast<char*>(sp.y) + (live ? row : 0) * (long long)sp.cols * TO::kBytes;

    float v[VPT][E];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int j = i * RT + t;
        if (live && j < nvec) {
            VecIn<TI>::load(xr + (long long)j * E * TI::kBytes, v[i]);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) v[i][e] = -INFINITY;
        }
    }

    // pass 1 over the slice: its maximum, then its exponentials and their sum
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int e = 0; e < E; ++e) m = fmaxf(m, v[i][e]);
    const float mref = (m == -INFINITY) ? 0.f : m;
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            v[i][e] = __builtin_amdgcn_exp2f((v[i][e] - mref) * kSmLog2e);
            if (e & 1) l1 += v[i][e];
            else l0 += v[i][e];
        }
    const float m_slice = m;
    float l = l0 + l1;

    // the row's state: lanes, then the waves of the row in a fixed order
    sm_wave_merge(m, l);
    if constexpr (WPR > 1) {
        if ((tid & 63) == 0) {
            s_m[grp][wave_in_row] = m;
            s_l[grp][wave_in_row] = l;
        }
        __syncthreads();
        m = s_m[grp][0];
        l = s_l[grp][0];
#pragma unroll
        for (int w = 1; w < WPR; ++w) sm_merge(m, l, s_m[grp][w], s_l[grp][w]);
    }

    // pass 2: y = e^(x - m_slice) * e^(m_slice - m) / l
    const bool dead = !(l > 0.f);
    const float s = dead ? 0.f : sm_rescale(m_slice, m) / l;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int j = i * RT + t;
        if (live && j < nvec) store_scaled<TO, E>(yr + (long long)j * E * TO::kBytes, v[i], s);
    }
    if (live && t == 0 && sp.lse) sp.lse[row] = dead ? -INFINITY : m + __builtin_amdgcn_logf(l) * kLn2;
}

// ---------------------------------------------------------------- resident rows, registers + LDS

// Workgroups of NT threads (1024, or 768 where 168 registers per thread
// hold more of the row than 128 do), one row at a time. Thread t holds
// vectors j = i*NT + t of its row for i < VPT in registers and for
// VPT <= i < VPT + VLDS in LDS, at byte ((i - VPT)*NT + t)*16 of the
// workgroup's buffer: a wave's LDS DMA writes 64 consecutive 16-byte slots,
// so each thread reads back only what its own wave loaded (no barrier needed
// for that), and consecutive lanes read consecutive 16-byte slots (no bank
// conflicts). The LDS part is read twice (maximum and sum, then output) and
// its exponentials are recomputed on the second read instead of being
// stored.
//
// The LDS part leaves room for one such workgroup per compute unit, so the
// grid is at most one per compute unit and each workgroup walks the rows
// blockIdx.x, blockIdx.x + gridDim.x, ... As soon as a thread has written
// out one of its vectors of row r, it starts loading the same vector of its
// next row into the register or LDS slot just freed: the stores of one row
// and the loads of the next are in flight together, instead of each
// workgroup's memory traffic stopping between rows.
template <typename TI, typename TO, int NT, int VPT, int VLDS>
__global__ __launch_bounds__(NT) void softmax_resident_lds_kernel(SoftmaxParams sp) {
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(NT % 256 == 0, "whole waves on every SIMD");
    constexpr int E = VecIn<TI>::kN;
    constexpr int NW = NT / 64;
    __shared__ __attribute__((aligned(1024))) char s_x[VLDS * NT * 16];
    // per-wave states by row parity: a wave that runs ahead writes the other
    // half while slower waves still read this row's
    __shared__ float s_m[2][NW], s_l[2][NW];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int nvec = sp.cols / E;
    const long long xrow_bytes = (long long)sp.cols * TI::kBytes;
    const long long yrow_bytes = (long long)sp.cols * TO::kBytes;

    // Buffer resources over one row, addressed by per-lane byte offsets only
    // (the hardware's range check covers the per-lane offset, not a scalar
    // one): vector j of x at j * 16. Vectors past the end of the row fall
    // outside the resource (read as zero, stores dropped) and are excluded
    // from the maximum and the sum by j < nvec.
    auto x_rsrc = [&](long long row) {
        return __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const char*>(sp.x) + row * xrow_bytes), 0, nvec * 16, kBufferFlags);
    };
    auto y_rsrc = [&](long long row) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(reinterpret_cast<char*>(sp.y) + row * yrow_bytes), 0,
                                                 nvec * E * TO::kBytes, kBufferFlags);
    };
    // Per-lane byte offsets of vector i: xoff + i*NT*16 (x) and
    // yoff + i*NT*E*size (y), where yoff = xoff * E*size/16 (the same register
    // when input and output elements have the same size). The per-row loop
    // below makes xoff opaque at the start of each row, so those sums are
    // formed where they are used instead of being hoisted out of the loop and
    // held in registers throughout.
    constexpr u32 kYScale = (u32)(E * TO::kBytes) / 16u;
    static_assert(kYScale * 16u == (u32)(E * TO::kBytes), "whole output vectors");
    u32 xoff = (u32)t * 16u;
    auto load_lds = [&](__amdgpu_buffer_rsrc_t rx, int k) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (FA_LDS void*)(s_x + (k * NT + wave * 64) * 16), 16,
                                                 xoff + (u32)((VPT + k) * NT) * 16u, 0, 0, 0);
    };
    // A register vector arrives as its raw 16 bytes in the first four words
    // of its float slots and is widened in place before use (the slots are
    // its own: the next row's vector i takes the registers of this row's
    // vector i as soon as that one is written out).
    auto load_reg = [&](__amdgpu_buffer_rsrc_t rx, int i, float* vi) {
        const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff + (u32)(i * NT) * 16u, 0, 0);
#pragma unroll
        for (int w = 0; w < 4; ++w) vi[w] = __uint_as_float(u[w]);
    };
    auto lds_vec = [&](int k, float* w) {
        const int j = (VPT + k) * NT + t;
        if (j < nvec) {
            VecIn<TI>::load_lds((const FA_LDS char*)s_x + (k * NT + t) * 16, w);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) w[e] = -INFINITY;
        }
    };

    long long row = blockIdx.x;
    float v[VPT][E];
    {
        const __amdgpu_buffer_rsrc_t rx = x_rsrc(row);
        // LDS part first, so its loads are in flight while the register part loads
#pragma unroll
        for (int k = 0; k < VLDS; ++k) load_lds(rx, k);
#pragma unroll
        for (int i = 0; i < VPT; ++i) load_reg(rx, i, v[i]);
    }
    for (int par = 0;; par ^= 1) {
        asm volatile("" : "+v"(xoff));
        const u32 yoff = xoff * kYScale;
        const long long next = row + gridDim.x;
        const bool has_next = next < sp.rows;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const u32x4 u = {__float_as_uint(v[i][0]), __float_as_uint(v[i][1]), __float_as_uint(v[i][2]),
                             __float_as_uint(v[i][3])};
            VecIn<TI>::cvt(u, v[i]);
            if (!(i * NT + t < nvec)) {
#pragma unroll
                for (int e = 0; e < E; ++e) v[i][e] = -INFINITY;
            }
        }
        wait_vmcnt0();  // this wave's LDS DMA of the row has landed too

        // the slice's maximum over both parts, then its exponentials and their sum
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < VPT; ++i)
#pragma unroll
            for (int e = 0; e < E; ++e) m = fmaxf(m, v[i][e]);
        // (the LDS loops stay rolled: one vector in flight keeps the register
        // part's budget)
#pragma clang loop unroll(disable)
        for (int k = 0; k < VLDS; ++k) {
            float w[E];
            lds_vec(k, w);
#pragma unroll
            for (int e = 0; e < E; ++e) m = fmaxf(m, w[e]);
        }
        const float mref = (m == -INFINITY) ? 0.f : m;
        float l0 = 0.f, l1 = 0.f;
#pragma unroll
        for (int i = 0; i < VPT; ++i)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                v[i][e] = __builtin_amdgcn_exp2f((v[i][e] - mref) * kSmLog2e);
                if (e & 1) l1 += v[i][e];
                else l0 += v[i][e];
            }
#pragma clang loop unroll(disable)
        for (int k = 0; k < VLDS; ++k) {
            float w[E];
            lds_vec(k, w);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = __builtin_amdgcn_exp2f((w[e] - mref) * kSmLog2e);
                if (e & 1) l1 += x;
                else l0 += x;
            }
        }
        const float m_slice = m;
        float l = l0 + l1;

        // the row's state: lanes, then the waves in a fixed order
        sm_wave_merge(m, l);
        if (lane == 0) {
            s_m[par][wave] = m;
            s_l[par][wave] = l;
        }
        __syncthreads();
        m = s_m[par][0];
        l = s_l[par][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) sm_merge(m, l, s_m[par][w], s_l[par][w]);

        // output, y = e^(x - m_slice) * e^(m_slice - m) / l, each vector's
        // slot refilled with the next row's vector once it is written
        const bool dead = !(l > 0.f);
        const float sc = dead ? 0.f : sm_rescale(m_slice, m) / l;
        const __amdgpu_buffer_rsrc_t ry = y_rsrc(row);
        const __amdgpu_buffer_rsrc_t rn = x_rsrc(has_next ? next : row);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            store_scaled_buf<TO, E>(ry, yoff + (u32)(i * NT) * (E * TO::kBytes), v[i], sc);
            if (has_next) load_reg(rn, i, v[i]);
        }
#pragma clang loop unroll(disable)
        for (int k = 0; k < VLDS; ++k) {
            float w[E];
            lds_vec(k, w);
#pragma unroll
            for (int e = 0; e < E; ++e) w[e] = __builtin_amdgcn_exp2f((w[e] - mref) * kSmLog2e);
            store_scaled_buf<TO, E>(ry, yoff + (u32)((VPT + k) * NT) * (E * TO::kBytes), w, sc);
            if (has_next) {
                wait_lgkmcnt0();  // the wave's read of slot k is done before the DMA refills it
                load_lds(rn, k);
            }
        }
        if (t == 0 && sp.lse) sp.lse[row] = dead ? -INFINITY : m + __builtin_amdgcn_logf(l) * kLn2;
        if (!has_next) break;
        row = next;
    }
#endif
}

// ---------------------------------------------------------------- streamed rows

// One workgroup of NT threads per row, any length. VEC: the row is a whole
// number of 16-byte vectors; otherwise elements are read one at a time.
template <typename TI, typename TO, int NT, bool VEC>
__global__ __launch_bounds__(NT) void softmax_stream_kernel(SoftmaxParams sp) {
    constexpr int E = VEC ? VecIn<TI>::kN : 1;
    constexpr int U = 4;  // vectors in flight per thread per step
    __shared__ float s_m[NT / 64], s_l[NT / 64];

    const int t = threadIdx.x;
    const long long row = blockIdx.x;
    const int cols = sp.cols;
    const int nvec = cols / E;
    const char* xr = reinterpret_cast<const char*>(sp.x) + row * (long long)cols * TI::kBytes;
    char* yr = reinterpret_cast<char*>(sp.y) + row * (long long)cols * TO::kBytes;

    auto load = [&](int j, float* v) {
        if constexpr (VEC) VecIn<TI>::load(xr + (long long)j * E * TI::kBytes, v);
        else v[0] = VecIn<TI>::load1(xr + (long long)j * TI::kBytes);
    };

    // pass 1: running (m, l) of this thread's vectors, one update per vector
    float m = -INFINITY, l = 0.f;
    for (int j0 = t; j0 < nvec; j0 += U * NT) {
        float v[U][E];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * NT;
            if (j < nvec) {
                load(j, v[u]);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) v[u][e] = -INFINITY;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vm = -INFINITY;
#pragma unroll
            for (int e = 0; e < E; ++e) vm = fmaxf(vm, v[u][e]);
            const float mn = fmaxf(m, vm);
            const float ref = (mn == -INFINITY) ? 0.f : mn;
            float add = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) add += __builtin_amdgcn_exp2f((v[u][e] - ref) * kSmLog2e);
            l = l * sm_rescale(m, ref) + add;
            m = mn;
        }
    }

    sm_wave_merge(m, l);
    if constexpr (NT > 64) {
        if ((t & 63) == 0) {
            s_m[t >> 6] = m;
            s_l[t >> 6] = l;
        }
        __syncthreads();
        m = s_m[0];
        l = s_l[0];
#pragma unroll
        for (int w = 1; w < NT / 64; ++w) sm_merge(m, l, s_m[w], s_l[w]);
    }
    const bool dead = !(l > 0.f);
    const float inv = dead ? 0.f : 1.f / l;
    const float mref = dead ? 0.f : m;

    // pass 2: y = e^(x - m) / l
    for (int j0 = t; j0 < nvec; j0 += U * NT) {
        float v[U][E];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * NT;
            if (j < nvec) load(j, v[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * NT;
            if (j < nvec) {
#pragma unroll
                for (int e = 0; e < E; ++e) v[u][e] = __builtin_amdgcn_exp2f((v[u][e] - mref) * kSmLog2e);
                if constexpr (VEC) store_scaled<TO, E>(yr + (long long)j * E * TO::kBytes, v[u], inv);
                else store1<TO>(yr + (long long)j * TO::kBytes, v[u][0] * inv);
            }
        }
    }
    if (t == 0 && sp.lse) sp.lse[row] = dead ? -INFINITY : m + __builtin_amdgcn_logf(l) * kLn2;
}

}  // namespace fa
