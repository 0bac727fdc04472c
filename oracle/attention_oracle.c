/*
 * Attention forward oracle: plain, slow, obviously correct, float64.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it. It shares no code with the HIP library.
 *
 * What it computes (the definition the tiled method reproduces up to rounding,
 * per the worked proofs on "La recurrencia del online softmax", section
 * "Demostración de corrección", and "Online Softmax 算法详解" section 2.1):
 *
 *   for every (b, h, i):
 *     A_i = { j : (causal == 0 or j <= i) and (mask == NULL or mask[b][j] != 0) }
 *     if A_i is empty:  O_i = 0, LSE_i = -inf, fully_masked_i = 1
 *       (the all-masked convention of "Online Softmax 算法详解" sections 7.2-7.3)
 *     else, in float64 with every input value upcast exactly:
 *       s_j  = scale * sum_t q[i][t] * k[j][t]                 for j in A_i
 *       pass 1: m  = max_j s_j
 *       pass 2: l  = sum_j exp(s_j - m)
 *       pass 3: p_j = exp(s_j - m) / l;  O_i = sum_j p_j * v[j];  LSE_i = m + ln(l)
 *
 * This is the safe three-pass softmax of "在线Softmax算法解析" section 1.1 and
 * "Online Softmax 算法详解" section 2.1, applied to one row of Q K^T, followed
 * by the weighted sum of V rows of "在线Softmax算法解析" section 3.1; the LSE is
 * the log-sum-exp of "Online Softmax 算法详解" section 8.1 in natural log.
 *
 * Inputs are float32 arrays: every bf16, fp16 or fp32 input value is exactly
 * representable in float32 and then in float64, so nothing is rounded before
 * the arithmetic. Layout: q, k, v are [B][H][N][d] row-major; mask is [B][N].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int allowed(const unsigned char* mask, int b, int N, int causal, long i, long j) {
    if (causal && j > i) return 0;
    if (mask && mask[(long)b * N + j] == 0) return 0;
    return 1;
}

/* One output row. s is caller scratch of N doubles. */
static void one_row(const float* q, const float* k, const float* v, const unsigned char* mask,
                    int B, int H, int N, int d, double scale, int causal, long long row,
                    double* s, double* o, double* lse, unsigned char* fully_masked) {
    (void)B;
    long long bh = row / N;
    long i = (long)(row % N);
    int b = (int)(bh / H);
    const float* qi = q + row * (long long)d;
    const float* kb = k + bh * (long long)N * d;
    const float* vb = v + bh * (long long)N * d;

    long count = 0;
    for (long j = 0; j < N; j++) {
        if (!allowed(mask, b, N, causal, i, j)) continue;
        double dot = 0.0;
        for (int t = 0; t < d; t++) dot += (double)qi[t] * (double)kb[(long long)j * d + t];
        s[j] = scale * dot;
        count++;
    }
    for (int t = 0; t < d; t++) o[t] = 0.0;
    if (count == 0) {
        *lse = -INFINITY;
        *fully_masked = 1;
        return;
    }
    /* pass 1: the row maximum */
    double m = -INFINITY;
    for (long j = 0; j < N; j++)
        if (allowed(mask, b, N, causal, i, j) && s[j] > m) m = s[j];
    /* pass 2: the normaliser relative to that maximum */
    double l = 0.0;
    for (long j = 0; j < N; j++)
        if (allowed(mask, b, N, causal, i, j)) l += exp(s[j] - m);
    /* pass 3: probabilities and the weighted sum of value rows */
    for (long j = 0; j < N; j++) {
        if (!allowed(mask, b, N, causal, i, j)) continue;
        double p = exp(s[j] - m) / l;
        const float* vj = vb + (long long)j * d;
        for (int t = 0; t < d; t++) o[t] += p * (double)vj[t];
    }
    *lse = m + log(l);
    *fully_masked = 0;
}

/*
 * Computes the rows listed in `rows` (flat indices (b*H + h)*N + i), or every
 * row when rows == NULL (then nrows must equal B*H*N). Outputs are packed in
 * the order of `rows`: o is [nrows][d], lse and fully_masked are [nrows].
 * nthreads <= 0 uses the OpenMP default. Returns 0, or -1 on bad arguments,
 * -2 on allocation failure.
 */
int oracle_attention_rows(const float* q, const float* k, const float* v,
                          const unsigned char* mask, int B, int H, int N, int d,
                          double scale, int causal, const long long* rows, long long nrows,
                          double* o, double* lse, unsigned char* fully_masked, int nthreads) {
    if (!q || !k || !v || !o || !lse || !fully_masked) return -1;
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return -1;
    long long total = (long long)B * H * N;
    if (!rows && nrows != total) return -1;
    int err = 0;
    int team = 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    team = omp_get_max_threads();
#else
    (void)nthreads;
#endif
    /* one row of scores per thread, allocated before the parallel region so
     * that every thread of the team reaches the worksharing loop */
    double* scratch = (double*)malloc(sizeof(double) * (size_t)N * (size_t)team);
    if (!scratch) return -2;
#pragma omp parallel num_threads(team)
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double* s = scratch + (size_t)tid * (size_t)N;
#pragma omp for schedule(dynamic, 1)
        for (long long r = 0; r < nrows; r++) {
            long long row = rows ? rows[r] : r;
            if (row < 0 || row >= total) {
#pragma omp atomic write
                err = -1;
                continue;
            }
            one_row(q, k, v, mask, B, H, N, d, scale, causal, row, s,
                    o + r * (long long)d, lse + r, fully_masked + r);
        }
    }
    free(scratch);
    return err;
}

/* Number of threads the OpenMP runtime would use (for reporting). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
