// Attention forward with online softmax for gfx950 (MI355X), FP8 E4M3 inputs.
//
// Q, K and V are OCP E4M3 values (the format gfx950's MFMA reads), each with
// a per-tensor float32 descale: the real input is value * descale. The loop is
// the 16-bit kernel's (attn_fwd_kernel.h) with three changes:
//
//   * products run on v_mfma_scale_f32_32x32x64_f8f6f4 (block scales set to
//     1): S^T = K Q^T contracts 64 d values per instruction, O^T += V^T P^T
//     64 keys, so a key tile is 64 keys and one instruction covers it per
//     32-wide block of d. The instruction pairs operand byte b of lane half h
//     in A with byte b of lane half h in B (checked on the GPU), so any
//     ordering of the contraction index that both operands share is valid.
//   * P is stored as E4M3 for the P V product, and E4M3 keeps only 3
//     mantissa bits with subnormals below 2^-6. As in "Online Softmax 算法详解"
//     section 6 ("FP8 Max_offset"), the exponent gets + MAXOFF (8) before
//     exp2, P' = 2^(s*c - m*c + 8) = 256 P in [0, 256], which moves the range
//     of P into E4M3's normal range. The running sum l' is taken from the
//     float32 P' and compensated at the end, l = l' / 2^MAXOFF, so the LSE is
//     unchanged; O = acc / l' needs no further factor because acc carries the
//     same 2^MAXOFF. P' must stay at most 448, E4M3's largest value, so a
//     growing row maximum cannot be left in P' for long (2^0.8 at most). The
//     growth goes instead into the instruction's E8M0 block scale of the P
//     operand, a per-lane power of two: O and the row sum keep a fixed
//     reference and are never multiplied on the way (see the online update
//     below); the 16-bit kernel's rescale of O by alpha is left for growth
//     beyond 2^64.
//   * V^T, the A operand of the P V product, is read from the row-major V
//     tile with ds_read_b64_tr_b8: within each 16-lane group, output byte b of
//     lane j is element j%8 of the 8-byte chunk addressed by lane 2b + j/8
//     (checked on the GPU). Lane l holds d = 32*db + l%32; the 32 keys of its
//     operand follow the S^T result layout of the lane's half, so P' packs
//     straight from the S^T registers (byte 16*kb + r = register r of key
//     block kb).
//
// Head dimension 128, four waves of 32 queries per workgroup.
#pragma once

#include "attn_common.h"

namespace fa {

struct ParamsFp8 {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const uint8_t* mask;  // [B][N] or nullptr
    int B, H, N;
    int n_qtiles;
    int xcd_remap;         // XcdMode: how workgroup ids spread over the 8 XCDs
    int head_group;       // heads whose query tiles are dealt together (>= 1)
    float c;              // scale * descale_q * descale_k * log2(e)
    float descale_v;
};

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Growth of the running maximum above the frame (log2 units) that P'' may
// carry before the next power of two moves into the block scale: P'' stays
// at most 2^(8 + 0.8) = 446, below E4M3's largest value 448.
constexpr float kFp8Headroom = 0.8f;
// Largest block-scale exponent before the frame itself moves: O and the row
// sum then hold at most 2^(64 + 8.8) times a sum of |V| rows, far inside fp32.
constexpr int kFp8MaxShift = 64;

// E4M3 x E4M3 -> float32, 32x32x64. The block scales are E8M0 (2^(e - 127)),
// one per lane for the 32 contraction elements the lane holds; A's are 2^0 and
// B's `scale_b` (one value per lane).
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c, int scale_b = 127) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, scale_b);
}

template <int D, int NW, typename TO, bool CAUSAL, bool MASK, int MAXOFF>
__global__ __launch_bounds__(NW * 64) void attn_fwd_fp8_kernel(ParamsFp8 p) {
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(D == 128, "head dim 128");
    constexpr int BC = 64;               // keys per tile
    constexpr int NT = NW * 64;
    constexpr int BR = NW * 32;
    constexpr int NKB = BC / 32;         // 32-key blocks per tile
    constexpr int NDM = D / 64;          // 64-wide d slices (QK contraction steps)
    constexpr int NDB = D / 32;          // 32-wide blocks of d in O^T
    constexpr int ROWB = D;              // bytes per row
    constexpr int CH = ROWB / 16;        // 16-byte chunks per row (8)
    constexpr int TILEB = BC * ROWB;
    constexpr int RPI = 1024 / ROWB;
    constexpr int LOADS = TILEB / 1024;
    constexpr int LPW = (LOADS + NW - 1) / NW;
    static_assert(CH == 8, "row layout");

    __shared__ __attribute__((aligned(1024))) char buf0[2 * TILEB];
    __shared__ __attribute__((aligned(1024))) char buf1[2 * TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int hh = lane >> 5;

    int split, bh, qt;  // workgroup -> (one key range, batch*head, query tile), as in the forward
    schedule(blockIdx.x, gridDim.x, p.n_qtiles, p.B * p.H, 1, p.head_group, p.xcd_remap, &split, &bh, &qt);
    const int b = bh / p.H;
    const int N = p.N;
    const int q0 = qt * BR;
    const int qw0 = q0 + wave * 32;

    const size_t head = (size_t)bh * (size_t)N * D;
    const char* qg = reinterpret_cast<const char*>(p.q) + head;
    const char* kg = reinterpret_cast<const char*>(p.k) + head;
    const char* vg = reinterpret_cast<const char*>(p.v) + head;

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

    // Q^T as the B operand of slice m: lane l holds query l%32 and
    // d = 64m + 32*(l/32) .. +31 (32 bytes).
    i32x8 qop[NDM];
    {
        const int qr = min(qw0 + col, N - 1);
        const char* src = qg + (size_t)qr * ROWB + hh * 32;
#pragma unroll
        for (int m = 0; m < NDM; ++m) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(src + m * 64);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(src + m * 64 + 16);
            qop[m] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                           (int)hi[3]};
        }
    }

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    float m_run = -INFINITY;  // running row maximum, raw q.k units
    float frame = -INFINITY;  // reference of acc and l_run, log2 units
    float l_run = 0.f;        // this lane's share of the running sum of 2^(s*c - frame + MAXOFF)
    const float c = p.c;
    const bool wave_live = qw0 < N;
    const int qq = qw0 + col;

    // K operand: row 32*kb + col, logical chunks 4m + 2*hh and +1. The
    // per-lane offsets within a tile are computed once, so both buffers and
    // both key blocks read through the same registers with the rest in the
    // instruction's constant offset.
    const int sw_col = swz<CH>(col);
    u32 k_off[NDM][2];
#pragma unroll
    for (int m = 0; m < NDM; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j) k_off[m][j] = (u32)(col * ROWB + (((4 * m + 2 * hh + j) ^ sw_col) << 4));
    // V^T by 8-bit transpose reads. Lane l of 16-lane group g (= l/16,
    // j = l%16) supplies, for output byte b' = j/2, the chunk of tile row
    // 16t + 8(b'/4) + 4*(g/2) + b'%4 (read t = 0..3) at d = 32db + 16(g%2) +
    // 8(j%2). The row's swizzle does not depend on t.
    u32 v_off[NDB];
    {
        const int g = lane >> 4, j = lane & 15, bp = j >> 1;
        const int rowlane = 8 * (bp >> 2) + 4 * (g >> 1) + (bp & 3);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int chunk = 2 * db + (g & 1);
            v_off[db] = (u32)(rowlane * ROWB + ((chunk ^ swz<CH>(rowlane)) << 4) + 8 * (j & 1));
        }
    }

    auto compute_tile = [&](int tile, const char* buf) {
        const int k0 = kv_begin + tile * BC;
        if (!wave_live || (CAUSAL && k0 > qw0 + 31)) return;
        const FA_LDS char* kt = (const FA_LDS char*)buf;
        const FA_LDS char* vt = (const FA_LDS char*)buf + TILEB;

        // ---- S^T = K_j Q^T
        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
        for (int m = 0; m < NDM; ++m) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const FA_LDS char* blk = kt + kb * 32 * ROWB;
                const u32x4 lo = *reinterpret_cast<const FA_LDS u32x4*>(blk + k_off[m][0]);
                const u32x4 hi = *reinterpret_cast<const FA_LDS u32x4*>(blk + k_off[m][1]);
                const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                s[kb] = mfma_fp8(a, qop[m], s[kb]);
            }
        }

        // ---- masks (register r of block kb is key k0 + 4*hh + kb*32 + 8*(r/4) + r%4)
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

        // ---- online update with the FP8 offset. The accumulators stay in a
        // fixed frame F (log2 units: the first maximum the row sees), and the
        // growth of the running maximum above it, g = M*c - F, is split into
        // an integer k = max(0, ceil(g - kFp8Headroom)) and the rest: P is
        // formed as P'' = 2^(s*c - F - k + MAXOFF), at most 2^(MAXOFF +
        // headroom), and the factor 2^k is applied by the P V instruction's
        // E8M0 block scale of the P operand (lane l's scale covers its query's
        // 32 keys) and to the row sum by ldexp, exactly. The frame moves (a
        // rescale of O and l by 2^-k) only when k would pass kFp8MaxShift.
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = pair_max(mx);
        m_run = fmaxf(m_run, mx);
        const float mc = m_run * c;                  // -inf while the row has no allowed key
        if (frame == -INFINITY) frame = mc;          // the first key the row sees sets the frame
        const float g = mc - frame;                  // NaN while both are -inf
        int k = g > kFp8Headroom ? (int)__builtin_ceilf(g - kFp8Headroom) : 0;
        if (__builtin_amdgcn_ballot_w64(k > kFp8MaxShift) != 0) {
            // move the frame up by k: O and l scale by 2^-k, exactly
            l_run = __builtin_ldexpf(l_run, -k);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[db][r] = __builtin_ldexpf(acc[db][r], -k);
            frame += (float)k;
            k = 0;
        }
        const float ref = ((frame == -INFINITY) ? 0.f : frame + (float)k) - (float)MAXOFF;
        // the compiler's exponential/MFMA interleave schedule for the block
        // below, as in the 16-bit kernel (0.5-0.7% here, the same results)
        __builtin_amdgcn_iglp_opt(2);
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
        l_run += __builtin_ldexpf(rs0 + rs1, k);
        const int pscale = 127 + k;  // E8M0 2^k

        // ---- P'^T as E4M3: byte 16*kb + r holds register r of block kb. The
        // first conversion of a word writes its low half and keeps the high
        // half, which the second overwrites; starting from the bits of an
        // input that is dead afterwards lets it convert in place.
        i32x8 pb;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int kb = w >> 2, r0 = 4 * (w & 3);
            int x = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][r0], s[kb][r0 + 1], __float_as_int(s[kb][r0]), false);
            x = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][r0 + 2], s[kb][r0 + 3], x, true);
            pb[w] = x;
        }

        // ---- O^T += V_j^T P'^T, 64 keys per instruction
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            i32x8 a;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (FA_LDS i32x2*)(vt + t * 16 * ROWB + v_off[db]));
                a[2 * t] = r2[0];
                a[2 * t + 1] = r2[1];
            }
            acc[db] = mfma_fp8(a, pb, acc[db], pscale);
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

    // ---- finalize: l = l' / 2^MAXOFF in the frame's units for the LSE;
    // O = acc / l' * descale_v
    const float l_tot = pair_sum(l_run);
    const bool dead = !(l_tot > 0.f);
    const float inv = dead ? 0.f : p.descale_v / l_tot;
    const float lse = dead ? -INFINITY : (frame + __builtin_amdgcn_logf(l_tot) - (float)MAXOFF) * kLn2;
    if (qq < N) {
        char* orow = reinterpret_cast<char*>(p.o) + (head + (size_t)qq * D) * TO::kBytes;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * db + 8 * g + 4 * hh;
                const float v4[4] = {acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
                store_row4<TO>(orow + d0 * TO::kBytes, v4, inv);
            }
        if (hh == 0) p.lse[(size_t)bh * N + qq] = lse;
    }
#endif
}

}  // namespace fa
