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

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_DTYPE_F32 = 0,   /* IEEE float32 */
    FA_DTYPE_BF16 = 1,  /* bfloat16 */
    FA_DTYPE_F16 = 2    /* IEEE float16 */
} fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = -1,      /* a required pointer is NULL */
    FA_ERR_SHAPE = -2,     /* B, H or N <= 0, or a size overflows */
    FA_ERR_HEADDIM = -3,   /* d is not 64 or 128 */
    FA_ERR_DTYPE = -4,     /* unsupported (in_dtype, out_dtype) pair */
    FA_ERR_SCALE = -5,     /* scale <= 0, NaN or infinite */
    FA_ERR_ALIGN = -6,     /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
    FA_ERR_TILE = -7,      /* the requested tile configuration does not exist */
    FA_ERR_LAUNCH = -8     /* the HIP runtime rejected the kernel launch */
} fa_status;

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
           const uint8_t* key_padding_mask, int in_dtype, int out_dtype, void* stream);

/* fa_fwd_ex — fa_fwd with an explicit tile shape (NULL = default). Returns
 * FA_ERR_TILE if no kernel exists for that shape with these arguments. */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int N, int d, float scale, int causal,
              const uint8_t* key_padding_mask, int in_dtype, int out_dtype, void* stream,
              const fa_tile* tile);

/* fa_default_tile — the tile shape fa_fwd would use for these arguments.
 * Writes *out and returns FA_OK, or returns a negative fa_status. Host only. */
int fa_default_tile(int N, int d, int in_dtype, int out_dtype, int causal, int has_mask,
                    fa_tile* out);

/* fa_tile_supported — FA_OK if fa_fwd_ex accepts `tile` for (d, in_dtype,
 * out_dtype), FA_ERR_TILE otherwise. Host only, no HIP call. */
int fa_tile_supported(int d, int in_dtype, int out_dtype, const fa_tile* tile);

/* fa_strerror — a static, human-readable name for a status code. */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
