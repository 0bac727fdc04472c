/*
 * fa.h — C ABI of the MI355X (gfx950) attention forward with online softmax.
 *
 * Operation (the single-pass fused loop of "Online Softmax 算法详解" section
 * 2.3, with the block update of "在线Softmax算法解析" section 3.2 and the
 * finalisation of "Online Softmax 算法详解" section 4.7):
 *
 *   for every batch b, head h and query row i:
 *     A_i  = { j : (causal == 0 or j <= i) and (mask == NULL or mask[b][j] != 0) }
 *     S_ij = scale * sum_t Q[b][h][i][t] * K[b][h][j][t]          for j in A_i
 *     O[b][h][i][:] = sum_{j in A_i} softmax_j(S_i) * V[b][h][j][:]
 *     LSE[b][h][i]  = ln sum_{j in A_i} exp(S_ij)
 *   A row with A_i empty gets O = 0 and LSE = -inf exactly (the guards of
 *   "Online Softmax 算法详解" sections 7.1-7.3).
 *
 * The result is computed tile by tile: the keys are walked in blocks, each
 * query row keeps its running maximum, running normaliser and unnormalised
 * output, rescaled by exp(m_old - m_new) when the maximum grows, and divided
 * once at the end. Matrix products run on bf16/fp16 MFMA with float32
 * accumulation (float32 inputs use float32 MFMA); exp is evaluated as exp2
 * with log2(e) folded into the scale.
 *
 * Layout: Q, K, V and O are [B][H][N][d], row-major and contiguous, d
 * innermost. LSE is [B][H][N] float32. The key mask is [B][N] uint8.
 *
 * Ownership: every pointer is a device pointer owned by the caller. The
 * library allocates nothing, keeps no state between calls, and is safe to
 * call from several host threads at once.
 *
 * Asynchrony: the work is enqueued on `stream` (a hipStream_t; NULL means the
 * default stream) and the call returns without synchronising. A fault inside
 * the kernel surfaces at the caller's next synchronisation, not here.
 *
 * Errors: every argument is validated on the host before any HIP call, so an
 * invalid call touches no device state. Functions return FA_OK (0) or a
 * negative fa_status value; fa_strerror() names it.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_DTYPE_F32 = 0,   /* IEEE float32 */
    FA_DTYPE_BF16 = 1,  /* bfloat16 */
    FA_DTYPE_F16 = 2,   /* IEEE float16 */
    /* Not dtypes: these give the enum the range of a 32-bit int, so every
     * int a caller passes is a value the library may read and reject with
     * FA_ERR_DTYPE. */
    FA_DTYPE_RANGE_MIN_ = INT32_MIN,
    FA_DTYPE_RANGE_MAX_ = INT32_MAX
} fa_dtype_t;

/* HIP stream handle: the same typedef as <hip/hip_runtime_api.h> makes, so
 * this header needs no HIP include (C11 and C++ accept the repeated typedef). */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = -1,      /* a required pointer is NULL */
    FA_ERR_SHAPE = -2,     /* B, H or N <= 0, or a size overflows */
    FA_ERR_HEADDIM = -3,   /* d is not 64 or 128 */
    FA_ERR_DTYPE = -4,     /* unsupported (in_dtype, out_dtype) pair */
    FA_ERR_SCALE = -5,     /* scale <= 0, NaN or infinite */
    FA_ERR_ALIGN = -6,     /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
    FA_ERR_TILE = -7,      /* the requested tile configuration does not exist */
    FA_ERR_LAUNCH = -8,    /* the HIP runtime rejected the kernel launch */
    FA_ERR_SPLITS = -9,    /* num_splits outside [1, FA_MAX_SPLITS] */
    FA_ERR_WORKSPACE = -10, /* workspace NULL, not 16-byte aligned, or too small */
    FA_ERR_OFFSET = -11,    /* fa_fwd_fp8: max_offset is neither 0 nor 8 */
    FA_ERR_SCRATCH = -12    /* fa_fwd_splitkv_noalloc: the partials exceed FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

/* Largest number of key-range parts fa_fwd_splitkv accepts. */
#define FA_MAX_SPLITS 64

/* Tile shape: block_r query rows per workgroup, block_c keys per K/V tile
 * (the B_r and B_c of the tiling). 0 in a field selects the default. */
typedef struct {
    int block_r;
    int block_c;
} fa_tile;

/*
 * fa_fwd — attention forward.
 *   q, k, v   [B][H][N][d] in_dtype, device, 16-byte aligned
 *   o         [B][H][N][d] out_dtype, device, 16-byte aligned (written)
 *   lse       [B][H][N] float32, device (written; natural log; -inf on rows
 *             with no allowed key)
 *   B, H, N   batch, heads, sequence length (> 0; N is the length of both the
 *             query and the key sequence)
 *   d         head dimension: 64 or 128
 *   scale     multiplier of Q K^T (> 0, finite), usually 1/sqrt(d)
 *   causal    nonzero: query i sees keys j <= i only
 *   key_padding_mask  NULL, or [B][N] uint8 device: nonzero = key valid
 *             (attended), 0 = padded (never attended)
 *   in_dtype, out_dtype  (BF16, BF16), (BF16, F32), (F16, F16), (F16, F32)
 *             or (F32, F32)
 *   stream    hipStream_t to enqueue on, or NULL
 * Returns FA_OK or a negative fa_status.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal,
           const uint8_t* key_padding_mask, fa_dtype_t in_dtype, fa_dtype_t out_dtype,
           hipStream_t stream);

/* fa_fwd_ex — fa_fwd with an explicit tile shape. NULL or {0, 0} is the
 * library's choice for the shape (fa_default_tile); a zero in one field takes
 * that field from the base tile (128 x 32 for 16-bit d = 128, 256 x 64 for
 * 16-bit d = 64, 128 x 64 for fp32). Returns FA_ERR_TILE if no kernel exists
 * for that shape with these arguments. */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int N, int d, float scale, int causal,
              const uint8_t* key_padding_mask, fa_dtype_t in_dtype, fa_dtype_t out_dtype,
              hipStream_t stream, const fa_tile* tile);

/* fa_default_tile — the tile shape fa_fwd would use for these arguments:
 * for 16-bit inputs at d = 128, 256 x 64 when every workgroup has a long key
 * loop and the grid of 256-row tiles, G = B*H*ceil(N/256), holds about one to
 * four workgroups per CU (causal: N >= 8192 and 384 <= G <= 1024;
 * non-causal: N >= 4096 and 256 <= G <= 1024), else the base tile. Writes *out and returns FA_OK, or returns a negative fa_status
 * (FA_ERR_NULL, FA_ERR_SHAPE for B, H or N <= 0, FA_ERR_HEADDIM,
 * FA_ERR_DTYPE). Host only, no HIP call. */
int fa_default_tile(int B, int H, int N, int d, fa_dtype_t in_dtype, fa_dtype_t out_dtype,
                    int causal, int has_mask, fa_tile* out);

/* fa_tile_supported — FA_OK if fa_fwd_ex accepts `tile` for (d, in_dtype,
 * out_dtype), FA_ERR_TILE otherwise. Host only, no HIP call. */
int fa_tile_supported(int d, fa_dtype_t in_dtype, fa_dtype_t out_dtype, const fa_tile* tile);

/*
 * Split-KV forward: the keys of every query row are cut into num_splits
 * contiguous ranges, processed by independent workgroups, and the partial
 * results merged afterwards. Each part runs the same tiled online-softmax loop
 * over its own range and leaves its normalised output O_s and its LSE_s; the
 * merge rescales the parts to their common maximum and adds them, which is the
 * two-state merge of the online-softmax interview card (section 三, the
 * merge equations) taken over S states at once, exact because the merge is
 * associative and commutative ("La recurrencia del online softmax", practice
 * problem 4). In LSE form, with M = max_s LSE_s and w_s = exp(LSE_s - M):
 *   O = sum_s w_s O_s / sum_s w_s,   LSE = M + ln sum_s w_s.
 * A part with no allowed key has LSE_s = -inf and weight 0; a row whose every
 * part is empty gets O = 0 and LSE = -inf exactly, as in fa_fwd.
 *
 * The point is parallelism when B * H * ceil(N / block_r) workgroups cannot
 * fill the device (small batch, few heads, short N): each part is one more
 * workgroup. The result matches fa_fwd to rounding; only the order of the
 * float32 additions differs.
 *
 * Every query tile's keys are cut into num_splits parts, except under a
 * causal mask with 16-bit inputs when B * H * ceil(N / block_r) <= 256: there
 * query tile t sees (t + 1) * block_r keys and gets parts in proportion, each
 * of at most u * block_r keys for the smallest u that leaves the last tile at
 * most num_splits parts, so that every workgroup has about the same work.
 */

/* fa_splitkv_workspace_bytes — bytes of device workspace fa_fwd_splitkv needs:
 * num_splits * B*H*N * (d + 1) * 4 (float32 partial outputs [S][B*H*N][d]
 * followed by partial LSEs [S][B*H*N]). Returns 0 for invalid arguments
 * (same rules as fa_fwd_splitkv). Host only, no HIP call. */
size_t fa_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits);

/* fa_splitkv_num_splits — a split count for these sizes and mask. With
 * equal parts per query tile: the smallest count whose workgroups fill every
 * slot of the 256 compute units at once (3 resident workgroups per CU for the
 * 16-bit d = 128 kernel, 2 for the 16-bit d = 64 kernel and fp32 inputs at
 * d = 64, 1 for fp32 inputs at d = 128), capped so that every part keeps at
 * least four key tiles (one for fp32 inputs) and at 8 parts. With parts in
 * proportion to the causal extent (causal != 0, 16-bit inputs, at most 256
 * query tiles; see fa_fwd_splitkv): the smallest count whose workgroups reach
 * 9/16 of those slots, capped at 12 and at four key tiles per part of the
 * longest query tile. Returns the count (1..12) or a negative fa_status.
 * Host only, no HIP call. */
int fa_splitkv_num_splits(int B, int H, int N, int d, fa_dtype_t in_dtype, int causal);

/*
 * fa_fwd_splitkv — attention forward with the keys split into num_splits
 * parts, then merged. Arguments as fa_fwd, plus:
 *   num_splits       1 .. FA_MAX_SPLITS (1 is valid: one part, then the merge)
 *   workspace        device memory of at least
 *                    fa_splitkv_workspace_bytes(B, H, N, d, num_splits) bytes,
 *                    16-byte aligned, owned by the caller; its contents on
 *                    entry do not matter and are overwritten. Two calls that
 *                    share a workspace must be ordered (same stream, or an
 *                    event between them): concurrent use races.
 *   workspace_bytes  its size in bytes
 * The tile shape is the default one for (d, in_dtype). Enqueues two kernels
 * (the split attention pass, then the merge) on `stream`. Returns FA_OK or a
 * negative fa_status; nothing is launched on error.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* key_padding_mask, fa_dtype_t in_dtype, fa_dtype_t out_dtype,
                   int num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Size of the fixed device scratch behind fa_fwd_splitkv_noalloc: 64 MiB per
 * device (e.g. 8 parts of B*H*N = 8192 rows at d = 128 need 33.8 MB). */
#define FA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * fa_fwd_splitkv_noalloc — fa_fwd_splitkv without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). The split partials go
 * to a fixed scratch array of FA_NOALLOC_SCRATCH_BYTES that the library's code
 * object holds on every device it is loaded on, until the process ends; the
 * call itself allocates nothing. Arguments and result as fa_fwd_splitkv, on
 * the calling thread's current device (the device of `stream`).
 *   Returns FA_ERR_SCRATCH, before any HIP call, when
 *   fa_splitkv_workspace_bytes(B, H, N, d, num_splits) > FA_NOALLOC_SCRATCH_BYTES
 *   (use fewer parts, or fa_fwd_splitkv with a workspace), and FA_ERR_LAUNCH
 *   if the scratch cannot be resolved on the current device.
 * Every call on a device shares that device's scratch, which keeps the last
 * call's partials (nothing in it needs to start at zero): calls on one device
 * must be ordered (same stream, or an event between them); calls that overlap
 * race and give wrong results.
 */
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, float scale, int causal,
                           const uint8_t* key_padding_mask, fa_dtype_t in_dtype,
                           fa_dtype_t out_dtype, int num_splits, hipStream_t stream);

/*
 * fa_fwd_fp8 — attention forward with FP8 (OCP E4M3) Q, K, V.
 *
 * The inputs are E4M3 bytes with per-tensor float32 descales: the real
 * values are q * descale_q, k * descale_k, v * descale_v. The operation is
 * fa_fwd's with S = scale * descale_q * descale_k * (q . k) and
 * O = descale_v * sum_j softmax_j(S) v_j. Products run on gfx950's E4M3 MFMA
 * with float32 accumulation, and P is rounded to E4M3 for the P V product.
 * With max_offset = 8, the FP8 setting of "Online Softmax 算法详解" section 6,
 * P is formed as 2^(S log2(e) - m log2(e) + 8) = 256 P, which places it in
 * E4M3's normal range; the running sum is compensated (l = l' / 256) so the
 * LSE is exact, and the output needs no extra factor. max_offset = 0 forms P
 * in [0, 1] (the 16-bit setting) and is provided for comparison.
 *   q, k, v   [B][H][N][d] E4M3 bytes, device, 16-byte aligned
 *   o         [B][H][N][d] out_dtype (BF16, F16 or F32), 16-byte aligned
 *   lse       [B][H][N] float32 (natural log; -inf on rows with no key)
 *   d         128
 *   scale, descale_q, descale_k, descale_v  > 0 and finite
 *   causal, key_padding_mask, stream  as for fa_fwd
 *   max_offset  8 or 0
 * Returns FA_OK or a negative fa_status: FA_ERR_HEADDIM for d != 128,
 * FA_ERR_DTYPE for another out_dtype, FA_ERR_SCALE when scale or a descale is
 * not positive and finite, FA_ERR_OFFSET for another max_offset, and the
 * other codes as fa_fwd.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, float descale_q, float descale_k,
               float descale_v, int causal, const uint8_t* key_padding_mask, fa_dtype_t out_dtype,
               int max_offset, hipStream_t stream);

/*
 * Attention backward from the saved LSE. The forward keeps no N x N matrix,
 * so the scores are recomputed tile by tile and the probabilities recovered
 * from the LSE the forward returned, P = exp(scale * Q K^T - LSE) over the
 * allowed keys, with no second online pass ("Online Softmax 算法详解"
 * section 8.3; the online-softmax interview card, section 四, point ③). With
 * D_i = sum_t dO_it O_it the gradients are the chain rule through O = P V
 * and the row softmax:
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
 *   dQ = scale * dS K,  dK = scale * dS^T Q.
 * Masked keys receive dK = dV = 0; rows with no allowed key (LSE = -inf)
 * contribute nothing and receive dQ = 0. Products run on bf16/fp16 MFMA with
 * float32 accumulation; every gradient element is accumulated by one lane
 * and stored once (no atomics, deterministic).
 */

/* fa_bwd_workspace_bytes — device workspace fa_bwd needs: per (b, h), two
 * floats per query padded to a multiple of 64 queries,
 * B * H * ceil(N / 64) * 512 bytes. 0 for invalid sizes. Host only. */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

/*
 * fa_bwd — gradients of fa_fwd.
 *   q, k, v, o, dout  [B][H][N][d] in_dtype, device, 16-byte aligned; o is
 *             the forward's output (in the input dtype) and dout the
 *             gradient with respect to it
 *   lse       [B][H][N] float32: the forward's LSE (natural log; -inf on
 *             rows with no allowed key)
 *   dq, dk, dv  [B][H][N][d] grad_dtype, device, 16-byte aligned (written)
 *   B, H, N, d, scale, causal, key_padding_mask  as for fa_fwd (the same
 *             values the forward was called with)
 *   in_dtype  BF16 or F16;  grad_dtype  in_dtype or F32
 *   workspace device memory of at least fa_bwd_workspace_bytes(B, H, N)
 *             bytes, 16-byte aligned, owned by the caller, overwritten
 *   stream    hipStream_t, or NULL
 * Enqueues the per-row D and LSE kernel, then dK/dV and dQ (two kernels at
 * d = 128, one launch holding both at d = 64). Calls
 * that share a workspace must be ordered on the device. Returns FA_OK or a
 * negative fa_status; nothing is launched on error.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
           float scale, int causal, const uint8_t* key_padding_mask, fa_dtype_t in_dtype,
           fa_dtype_t grad_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_softmax_fwd — softmax of every row of a matrix, with the online
 * normaliser.
 *
 * For each row x (length cols): m = max_i x_i, l = sum_i exp(x_i - m),
 *   y_i = exp(x_i - m) / l,   lse = m + ln l.
 * This is the two-pass online softmax of "Online Softmax 算法详解" section 2.2:
 * pass 1 produces m and l together with the incremental update (a larger
 * maximum rescales the running sum by exp(m_old - m_new)), pass 2 writes y.
 * Partial states of parts of a row combine with the merge of the
 * online-softmax interview card (section 三). Entries equal to -inf are
 * masked (y = 0 there); a row with no finite entry gets y = 0 and lse = -inf
 * exactly. Arithmetic is float32 (exp as exp2 with log2(e) folded in).
 *
 *   x     [rows][cols] in_dtype, device, 16-byte aligned, row-major
 *   y     [rows][cols] out_dtype, device, 16-byte aligned (written). y may be
 *         x itself when in_dtype == out_dtype; any other overlap is undefined.
 *   lse   [rows] float32, device (written; natural log), or NULL
 *   rows  1 .. 2^31 - 1;  cols >= 1;  rows * cols <= 2^40
 *   in_dtype, out_dtype  as fa_fwd: (BF16, BF16), (BF16, F32), (F16, F16),
 *         (F16, F32), (F32, F32)
 *   stream  hipStream_t, or NULL
 * A row of at most 65536 (16-bit) or 32768 (fp32) elements whose length is a
 * multiple of 8 (16-bit) or 4 (fp32) elements is held in registers: x is read
 * from memory once. Other rows are streamed twice (one workgroup per row).
 * Returns FA_OK or a negative fa_status; nothing is launched on error.
 */
int fa_softmax_fwd(const void* x, void* y, float* lse, long long rows, int cols,
                   fa_dtype_t in_dtype, fa_dtype_t out_dtype, hipStream_t stream);

/* fa_strerror — a static, human-readable name for a status code. */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
