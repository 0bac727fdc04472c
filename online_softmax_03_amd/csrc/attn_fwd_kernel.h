// Attention forward with online softmax for gfx950 (MI355X), bf16/fp16 inputs.
//
// One workgroup owns B_r = 32*NW query rows of one (batch, head); each of its
// NW waves owns 32 of them. The workgroup walks the key/value sequence in
// tiles of B_c rows ("Online Softmax 算法详解" section 2.3: only K/V blocks are
// looped over; every query row keeps its own state, "在线Softmax算法解析"
// section 3.3). Per tile:
//
//   1. K_j and V_j land in LDS straight from HBM (buffer_load_dwordx4 ... lds,
//      16 bytes per lane, coalesced), double-buffered so the next tile's load
//      overlaps this tile's math. Rows past the end of the sequence fall
//      outside the buffer resource and read as zero.
//   2. S^T = K_j * Q^T on v_mfma_f32_32x32x16 (bf16/fp16 in, fp32 out). The
//      transposed product puts one query per lane column: lane l holds query
//      l%32 and 16 of the tile's 32 keys per 32-key block, the other 16 sit in
//      lane l^32. Row max and row sum are then in-lane reductions plus a single
//      v_permlane32_swap, instead of a 32-lane butterfly.
//   3. Mask (causal diagonal, key range, padded keys) by writing -inf.
//   4. Online update in raw score units with the scale folded into exp2
//      ("Online Softmax 算法详解" sections 4.3, 4.5, 5): each row keeps a
//      reference maximum m; with m_new = max(m, rowmax) the state is rescaled,
//      alpha = 2^((m - m_new)*c), l *= alpha, O *= alpha, m = m_new, and then
//      P = 2^(s*c - m*c) as one FMA plus v_exp_f32, l += sum P, with
//      c = scale*log2(e). The rescale is conditional, as in step 3 of
//      "在线Softmax算法解析" section 2.1, but with a margin: it runs only when
//      some row of the wave saw its maximum grow by more than kRescaleLog2
//      (in log2 units) since the last rescale. Until then P may exceed 1 by up
//      to 2^kRescaleLog2, which bf16, fp16 and the fp32 accumulators hold
//      easily, and the result is unchanged because any reference point gives
//      the same O/l (the shift invariance the pages' exactness proofs rest on).
//      The -inf guard of "Online Softmax 算法详解" section 7.1 uses 0 as the
//      subtrahend while m is still -inf.
//   5. P is rounded to bf16/fp16 in registers and fed straight back as the B
//      operand of O^T += V_j^T * P^T: the MFMA result layout of S^T matches the
//      operand layout up to a fixed permutation of keys inside each 16-key
//      group, and the V^T operand is read from the row-major V tile with
//      ds_read_b64_tr_b16 in that same key order. No LDS round trip for P.
//      The row sum l is accumulated from the fp32 P before rounding (as the
//      deferred row sum of "Online Softmax 算法详解" section 4.6 is) for bf16
//      inputs: summing the rounded values instead would put bf16's 2^-8
//      relative error straight into the LSE. For fp16 inputs it is taken from
//      the rounded P (2^-11 relative, an LSE error of at most 4.9e-4), two
//      values per v_dot2_f32_f16.
//
// After the last tile: the two lane halves' row sums are added (the deferred
// cross-lane reduce of "Online Softmax 算法详解" section 4.6), inv = 1/l with the
// l == 0 / NaN guard of section 7.2, O *= inv, LSE = (m*c + log2 l)*ln 2 with
// the -inf case of section 7.3, and O and LSE are stored.
#pragma once

#include "attn_common.h"

namespace fa {

// ---------------------------------------------------------------- kernel

// Waves per SIMD the 128 x 32 tile at d = 128 is held to in its split-KV and
// key-masked forms: three (at most 168 registers). The host sizes its split
// count by the workgroups a compute unit holds (resident_wgs_per_cu in
// fa_api.hip), and the masked forms would otherwise take 2-3 registers more
// than three waves allow. Its other forms stay well below the bound without
// it (and were 0.3% slower with it on the causal bf16 workload); the 256 x 64
// tile at d = 64 meets its count of two (at most 128 registers) by itself.
template <int D, int BC, int NW, bool SPLIT, bool MASK>
constexpr int min_waves_per_eu() {
    return (D == 128 && BC == 32 && NW == 4 && (SPLIT || MASK)) ? 3 : 1;
}

template <int D, int BC, int NW, typename TI, typename TO, bool CAUSAL, bool MASK, bool SPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(min_waves_per_eu<D, BC, NW, SPLIT, MASK>())))
void attn_fwd_kernel(Params p) {
    // The body uses device-only types (buffer resources), so the host pass,
    // which only needs the launch stub, does not see it.
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BC % 32 == 0 && BC >= 32 && BC <= 128, "key tile");
    static_assert(TI::kBytes == 2, "16-bit inputs (fp32 inputs use attn_fwd_f32_kernel)");
    constexpr int NT = NW * 64;
    constexpr int BR = NW * 32;          // query rows per workgroup
    constexpr int NKB = BC / 32;         // 32-key blocks per tile
    constexpr int NDC = D / 16;          // 16-wide slices of d (QK contraction steps)
    constexpr int NDB = D / 32;          // 32-wide blocks of d in O^T
    constexpr int EB = TI::kBytes;       // bytes per input element
    constexpr int ROWB = D * EB;         // bytes per row
    constexpr int CH = ROWB / 16;        // 16-byte chunks per row
    constexpr int TILEB = BC * ROWB;     // bytes per K or V tile
    constexpr int RPI = 1024 / ROWB;     // tile rows per 1 KB wave load
    constexpr int LOADS = TILEB / 1024;  // wave loads per tensor per tile
    constexpr int LPW = (LOADS + NW - 1) / NW;

    // Two tile buffers, each K then V. They are distinct objects (not one
    // array indexed by parity) so the compiler can see that this tile's LDS
    // reads never alias the next tile's in-flight DMA writes.
    __shared__ __attribute__((aligned(1024))) char buf0[2 * TILEB];
    __shared__ __attribute__((aligned(1024))) char buf1[2 * TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;  // query within the wave's 32
    const int hh = lane >> 5;   // which 16 of every 32 keys this lane holds

    // workgroup -> (key-range part, batch*head, query tile): every tile of a
    // head runs on one XCD, so the workgroups sharing its K/V share an L2, and
    // each XCD starts its longest tiles (largest causal extent) first
    // (schedule, work_item.h; causal split launches give every part about the
    // same number of key tiles, schedule_parts / locate_part).
    int split, n_parts, bh, qt;
    attn_schedule<SPLIT, CAUSAL>(p, &split, &n_parts, &bh, &qt);
    const int b = bh / p.H;
    const int N = p.N;
    const int q0 = qt * BR;
    const int qw0 = q0 + wave * 32;

    const size_t head = (size_t)bh * (size_t)N * D;
    const char* qg = reinterpret_cast<const char*>(p.q) + head * EB;
    const char* kg = reinterpret_cast<const char*>(p.k) + head * EB;
    const char* vg = reinterpret_cast<const char*>(p.v) + head * EB;

    // Keys [key_lo, key_hi) may be valid: the whole sequence, or the extent of
    // the key mask's valid entries. When those entries are contiguous (a
    // padding mask), the range test below is the whole mask; otherwise every
    // key is also looked up in the mask.
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

    // V halves of both buffers start at zero so that a row the DMA leaves
    // untouched can never inject a non-finite value into P*V.
    {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int off = tid * 16; off < TILEB; off += NT * 16) {
            *reinterpret_cast<FA_LDS u32x4*>((FA_LDS char*)buf0 + TILEB + off) = z;
            *reinterpret_cast<FA_LDS u32x4*>((FA_LDS char*)buf1 + TILEB + off) = z;
        }
        __syncthreads();
    }

    // DMA geometry. Wave load R of a tile fills bytes [R*1024, R*1024+1024):
    // lane s writes slot s, i.e. tile row R*RPI + s/CH at physical chunk s%CH,
    // which holds logical chunk (s%CH) ^ swz(row). lane_off[ii] is that row
    // and chunk as a byte offset from the tile's first row.
    u32 lane_off[LPW];
#pragma unroll
    for (int ii = 0; ii < LPW; ++ii) {
        const int R = wave + ii * NW;
        const int trow = R * RPI + lane / CH;
        lane_off[ii] = (u32)(trow * ROWB + (((lane % CH) ^ swz<CH>(trow)) * 16));
    }
    auto issue_tile = [&](int tile, char* buf) {
        const int k0 = kv_begin + tile * BC;
        const int bytes = (N - k0) * ROWB;  // rows past N are out of range: read as 0
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

    // Q^T as the B operand: lane l holds query l%32 and d = 16*dc + 8*(l/32)
    // .. +7 in qop[dc].
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
    float m_run = -INFINITY;  // reference row maximum, raw q.k units
    float l_run = 0.f;        // this lane's share of the running row sum
    const float c = p.c;
    const bool wave_live = qw0 < N;
    const int qq = qw0 + col;  // this lane's query

    // K operand rows are 32*kb + col: one chunk XOR per lane. The per-lane
    // offsets within a tile are computed once, like the V^T ones below, so
    // that both buffers read through the same registers with the buffer and
    // the key block in the instruction's constant offset.
    const int sw_col = swz<CH>(col);
    u32 k_off[NDC];
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) k_off[dc] = (u32)(col * ROWB + (((2 * dc + hh) ^ sw_col) << 4));
    // V^T transpose reads (16-bit path): within each 16-lane group, lane
    // 4r + c addresses tile row key0 + r at d offset dbase + 4c, where key0 =
    // 32kb + 16t + 8*half + 4*hh and dbase = 32db + 16*(group & 1). The XOR
    // pattern of those rows does not depend on kb or t, so each (db, half)
    // address is one per-lane offset plus a constant.
    const int tr_r = (lane & 15) >> 2;
    const int tr_c = lane & 3;
    const int tr_dsub = (lane >> 4) & 1;
    u32 v_off[NDB][2];
    {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int row = 8 * half + 4 * hh + tr_r;
                const int chunk = 4 * db + 2 * tr_dsub + (tr_c >> 1);
                v_off[db][half] = (u32)(row * ROWB + ((chunk ^ swz<CH>(row)) << 4) + (tr_c & 1) * 8);
            }
    }

    auto compute_tile = [&](int tile, const char* buf) {
        const int k0 = kv_begin + tile * BC;
        // Waves whose queries all precede this tile's first key have nothing to do.
        if (!wave_live || (CAUSAL && k0 > qw0 + 31)) return;
        const FA_LDS char* kt = (const FA_LDS char*)buf;
        const FA_LDS char* vt = (const FA_LDS char*)buf + TILEB;

        // ---- S^T = K_j Q^T
        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const u32x4 a = *reinterpret_cast<const FA_LDS u32x4*>(kt + kb * 32 * ROWB + k_off[dc]);
                s[kb] = mfma32x32x16<TI>(a, qop[dc], s[kb]);
            }
        }

        // ---- masks. Register r of block kb is key k0 + 4*hh + kb*32 +
        // 8*(r/4) + r%4; the constant part is compared against per-lane limits.
        const bool edge_lo = k0 < key_lo;
        const bool edge_hi = k0 + BC > kv_end;
        const bool diag = CAUSAL && (k0 + BC - 1 > qw0);
        if (edge_lo || edge_hi || diag || (MASK && mask_general)) {
            const int base = k0 + 4 * hh;
            int hi = min(key_hi, kv_end) - 1 - base;  // last allowed key, relative
            if (CAUSAL) hi = min(hi, qq - base);
            const int lo = key_lo - base;             // first allowed key, relative
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

        // ---- online softmax update
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = pair_max(mx);
        const float m_new = fmaxf(m_run, mx);
        // (m_new - m_run)*c is +inf on a row's first live tile (m_run = -inf)
        // and NaN while the row has seen only masked keys (no rescale needed).
        if (__builtin_amdgcn_ballot_w64((m_new - m_run) * c > kRescaleLog2) != 0) {
            // rows still at -inf (only masked keys so far) get alpha = 2^-inf = 0
            const float alpha =
                __builtin_amdgcn_exp2f(m_run * c - ((m_new == -INFINITY) ? 0.f : m_new * c));
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
            m_run = m_new;
        }
        const float ref = (m_run == -INFINITY) ? 0.f : m_run * c;
        // The compiler's exponential/MFMA interleave schedule for the block
        // below (exponentials, packing, P*V): it spreads the v_exp_f32 and
        // packing work between the P*V MFMAs instead of ahead of them. Not
        // with a key mask at d = 128, where it costs registers (the 64-key
        // tiles' masked forms grow by 40-50 of them) and gains nothing.
        if constexpr (!(D == 128 && MASK)) __builtin_amdgcn_iglp_opt(2);
        constexpr bool kSumRounded = std::is_same_v<TI, F16>;
        // Two chains for the row sum. The float32 sums start from their
        // first terms rather than from 0 (the same value: exp2 is never -0),
        // which saves an add per chain and tile.
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -ref));
                if constexpr (!kSumRounded) {
                    float& rs = (r & 1) ? rs1 : rs0;
                    rs = (kb == 0 && r < 2) ? s[kb][r] : rs + s[kb][r];
                }
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
        if constexpr (kSumRounded) {
            // fp16 inputs: the row sum is taken from the rounded P the P*V
            // product uses, two values per v_dot2_f32_f16 (half the adds).
            // fp16 keeps 11 significant bits, so each term is within 2^-11
            // of its float32 value and the sum within 2^-11 relative: an LSE
            // error of at most 4.9e-4. (bf16 keeps 8 significant bits, whose
            // 2^-8 would allow 3.9e-3, so the bf16 path sums the float32
            // values.)
            const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // through a scalar: a bit cast of the vector element
                        // expression itself reads the wrong word in this compiler
                        const u32 w = pb[kb][t][j];
                        const f16x2 pp = __builtin_bit_cast(f16x2, w);
                        if (j & 1) rs1 = __builtin_amdgcn_fdot2(pp, one, rs1, false);
                        else rs0 = __builtin_amdgcn_fdot2(pp, one, rs0, false);
                    }
        }
        l_run += rs0 + rs1;

        // ---- O^T += V_j^T P^T. Register j of the B operand above is key
        // 16t + 8(j/4) + 4*hh + j%4 of the block; the A operand must hold
        // V[that key][d = l%32] in the same slot. Two ds_read_b64_tr_b16
        // give it: after the transpose, lane i of a 16-lane group holds
        // V[key0 .. key0+3][dbase + i].
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rowc = (kb * 32 + t * 16) * ROWB;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const i16x4 lo =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(vt + rowc + v_off[db][0]));
                    const i16x4 hi =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(vt + rowc + v_off[db][1]));
                    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
                    const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
                    const u32x4 a = {lo2[0], lo2[1], hi2[0], hi2[1]};
                    acc[db] = mfma32x32x16<TI>(a, pb[kb][t], acc[db]);
                }
            }
        }
    };

    // Main loop, unrolled by two so each half names its buffer statically.
    if (n_tiles > 0) issue_tile(0, buf0);
    for (int it = 0; it < n_tiles; it += 2) {
        if (p.fair) {
            // Equal progress: a wave's issue priority falls with the share of
            // its tiles done, so the waves furthest behind issue first.
            const int quarter = (it * 4) / n_tiles;
            if (quarter == 0) __builtin_amdgcn_s_setprio(3);
            else if (quarter == 1) __builtin_amdgcn_s_setprio(2);
            else if (quarter == 2) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        }
        wait_vmcnt0();     // this wave's loads of tile `it` have landed
        __syncthreads();   // ... everyone's, and tile it-1 (buffer 1) is no longer read
        if (it + 1 < n_tiles) issue_tile(it + 1, buf1);
        compute_tile(it, buf0);
        if (it + 1 >= n_tiles) break;
        wait_vmcnt0();
        __syncthreads();
        if (it + 2 < n_tiles) issue_tile(it + 2, buf0);
        compute_tile(it + 1, buf1);
    }

    // ---- finalize and store
    const float l_tot = pair_sum(l_run);
    const bool dead = !(l_tot > 0.f);  // no allowed key (sum 0) or NaN
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
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace fa
