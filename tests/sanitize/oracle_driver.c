/*
 * Runs the float64 attention oracle (oracle/attention_oracle.c, included
 * whole) on small shapes under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every row, selected rows, masks with empty and full batches, causal and
 * not, one and several OpenMP threads, and the argument errors. Each result is
 * checked against a direct evaluation of the definition written here (naive
 * exp / sum, valid at these magnitudes). Exit status 0 when all agree.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/attention_oracle.c"

static unsigned long long rng = 88172645463325252ULL;
static double urand(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}

static int check(int B, int H, int N, int d, int causal, int use_mask, int threads) {
    const long long rows = (long long)B * H * N, n = rows * d;
    float* q = malloc(sizeof(float) * n);
    float* k = malloc(sizeof(float) * n);
    float* v = malloc(sizeof(float) * n);
    unsigned char* mask = use_mask ? malloc((size_t)B * N) : NULL;
    double* o = malloc(sizeof(double) * n);
    double* lse = malloc(sizeof(double) * rows);
    unsigned char* fm = malloc((size_t)rows);
    for (long long i = 0; i < n; i++) {
        q[i] = (float)(4 * urand() - 2);
        k[i] = (float)(4 * urand() - 2);
        v[i] = (float)(2 * urand() - 1);
    }
    if (mask) {
        for (int b = 0; b < B; b++)
            for (int j = 0; j < N; j++) mask[b * N + j] = b == 0 ? 0 : (b == 1 ? 1 : urand() < 0.5);
    }
    const double scale = 0.3;
    int bad = oracle_attention_rows(q, k, v, mask, B, H, N, d, scale, causal, NULL, rows, o, lse, fm, threads);
    for (long long r = 0; r < rows && !bad; r++) {
        const long long bh = r / N, i = r % N, b = bh / H;
        double l = 0.0, acc[64] = {0};
        for (long long j = 0; j < N; j++) {
            if ((causal && j > i) || (mask && !mask[b * N + j])) continue;
            double dot = 0.0;
            for (int t = 0; t < d; t++) dot += (double)q[r * d + t] * k[(bh * N + j) * d + t];
            const double e = exp(scale * dot);
            l += e;
            for (int t = 0; t < d; t++) acc[t] += e * v[(bh * N + j) * d + t];
        }
        if (l == 0.0) {
            if (!fm[r] || !isinf(lse[r]) || lse[r] > 0) bad = 1;
            for (int t = 0; t < d; t++)
                if (o[r * d + t] != 0.0) bad = 1;
        } else {
            if (fm[r] || fabs(lse[r] - log(l)) > 1e-12) bad = 1;
            for (int t = 0; t < d; t++)
                if (fabs(o[r * d + t] - acc[t] / l) > 1e-12) bad = 1;
        }
    }
    /* a selection of rows, in a shuffled order, equals the full result */
    long long sel[5] = {rows - 1, 0, rows / 2, 1 % rows, rows / 3};
    double o2[5 * 64], l2[5];
    unsigned char f2[5];
    if (!bad && oracle_attention_rows(q, k, v, mask, B, H, N, d, scale, causal, sel, 5, o2, l2, f2, threads)) bad = 1;
    for (int r = 0; r < 5 && !bad; r++) {
        if (f2[r] != fm[sel[r]] || !(l2[r] == lse[sel[r]])) bad = 1;
        for (int t = 0; t < d; t++)
            if (o2[r * d + t] != o[sel[r] * d + t]) bad = 1;
    }
    /* argument errors: out-of-range rows, missing outputs, bad sizes */
    long long wrong[2] = {0, rows};
    if (oracle_attention_rows(q, k, v, mask, B, H, N, d, scale, causal, wrong, 2, o2, l2, f2, threads) != -1) bad = 1;
    if (oracle_attention_rows(q, k, v, mask, B, H, N, d, scale, causal, NULL, rows + 1, o, lse, fm, threads) != -1)
        bad = 1;
    if (oracle_attention_rows(q, k, v, mask, B, H, N, d, scale, causal, NULL, rows, NULL, lse, fm, threads) != -1)
        bad = 1;
    if (oracle_attention_rows(q, k, v, mask, 0, H, N, d, scale, causal, NULL, 0, o, lse, fm, threads) != -1) bad = 1;
    free(q);
    free(k);
    free(v);
    free(mask);
    free(o);
    free(lse);
    free(fm);
    if (bad) fprintf(stderr, "mismatch at B=%d H=%d N=%d d=%d causal=%d mask=%d threads=%d\n", B, H, N, d, causal,
                     use_mask, threads);
    return bad;
}

int main(void) {
    int bad = 0;
    for (int causal = 0; causal < 2; causal++)
        for (int use_mask = 0; use_mask < 2; use_mask++)
            for (int threads = 1; threads <= 4; threads += 3) {
                bad |= check(4, 2, 9, 3, causal, use_mask, threads);
                bad |= check(3, 1, 33, 16, causal, use_mask, threads);
                bad |= check(1, 1, 1, 64, causal, use_mask, threads);
            }
    if (bad) return 1;
    printf("oracle: ok (threads reported %d)\n", oracle_max_threads());
    return 0;
}
