/*
 * Runs every function of the fp64 oracle on small seeded problems; built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by test_oracle_sanitized.py,
 * so that an out-of-bounds access or undefined behaviour in the oracle (which
 * produces every expected value the tests compare with) fails a test instead
 * of silently changing the expected values.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_pool(int bh, int N, int d, int B, int L, const double *x, double *pyr);
void oracle_select(int bh, int N, int d, int B, int L, int K, const double *pyr_q,
                   const double *pyr_k, int32_t *idx, double *relgap);
void oracle_attn_fwd(int bh, int N, int d, int B, int L, int K, int Le, double scale,
                     int drop_covered, const double *q, const double *k, const double *v,
                     const double *pyr_k, const double *pyr_v, const int32_t *idx, double *o,
                     double *lse);
void oracle_attn_bwd(int bh, int N, int d, int B, int L, int K, int Le, double scale,
                     int drop_covered, const double *q, const double *k, const double *v,
                     const double *pyr_k, const double *pyr_v, const int32_t *idx,
                     const double *dout, double *dq, double *dk, double *dv);
int oracle_transpose(int nb, int rows, int k, int cols, const int32_t *idx, int32_t *ptr,
                     int32_t *col);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double uniform(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double *filled(int64_t n)
{
    double *p = malloc((size_t)n * sizeof(double));
    for (int64_t i = 0; i < n; ++i)
        p[i] = uniform();
    return p;
}

int main(void)
{
    /* bh, N, B, L, K, Le, drop_covered */
    static const int shapes[][7] = {
        {2, 1024, 16, 2, 2, 1, 1},  /* 4 coarsest tokens */
        {2, 768, 16, 2, 2, 1, 1},   /* 3 coarsest tokens: a ragged dense tile */
        {3, 336, 16, 1, 5, 0, 0},   /* single level, 21 blocks, drop rule off */
        {1, 256, 16, 2, 16, 1, 1},  /* K = all blocks */
        {1, 16, 16, 1, 1, 0, 1},    /* one block */
        {1, 4096, 16, 3, 4, 2, 1},  /* three levels, two coarse levels */
        {1, 2368, 64, 1, 8, 0, 1},  /* blocks of 64, 37 blocks */
        {1, 2048, 16, 2, 32, 1, 0}, /* K = 32, drop rule off */
    };
    const int d = 64;
    for (unsigned si = 0; si < sizeof shapes / sizeof shapes[0]; ++si) {
        const int bh = shapes[si][0], N = shapes[si][1], B = shapes[si][2], L = shapes[si][3];
        const int K = shapes[si][4], Le = shapes[si][5], drop = shapes[si][6];
        int n[8], kl[8];
        int64_t pyr = 0, nidx = 0;
        for (int l = 1, span = B; l <= L; ++l, span *= B)
            n[l] = N / span;
        kl[L] = K < n[L] ? K : n[L];
        for (int l = L - 1; l >= 1; --l)
            kl[l] = K < kl[l + 1] * B ? K : kl[l + 1] * B;
        for (int l = 1; l <= L; ++l) {
            pyr += (int64_t)bh * n[l] * d;
            nidx += (int64_t)bh * n[l] * kl[l];
        }
        const int64_t tok = (int64_t)bh * N * d;
        double *q = filled(tok), *k = filled(tok), *v = filled(tok), *dout = filled(tok);
        double *pq = malloc((size_t)pyr * sizeof(double));
        double *pk = malloc((size_t)pyr * sizeof(double));
        double *pv = malloc((size_t)pyr * sizeof(double));
        int32_t *idx = malloc((size_t)nidx * sizeof(int32_t));
        int64_t rows = 0;
        for (int l = 1; l <= L; ++l)
            rows += (int64_t)bh * n[l];
        double *gap = malloc((size_t)rows * sizeof(double));
        oracle_pool(bh, N, d, B, L, q, pq);
        oracle_pool(bh, N, d, B, L, k, pk);
        oracle_pool(bh, N, d, B, L, v, pv);
        oracle_select(bh, N, d, B, L, K, pq, pk, idx, gap);
        double *o = malloc((size_t)tok * sizeof(double));
        double *lse = malloc((size_t)bh * N * sizeof(double));
        oracle_attn_fwd(bh, N, d, B, L, K, Le, 0.125, drop, q, k, v, pk, pv, idx, o, lse);
        double *dq = calloc((size_t)tok, sizeof(double));
        double *dk = calloc((size_t)tok, sizeof(double));
        double *dv = calloc((size_t)tok, sizeof(double));
        oracle_attn_bwd(bh, N, d, B, L, K, Le, 0.125, drop, q, k, v, pk, pv, idx, dout, dq, dk, dv);
        int32_t *ptr = malloc((size_t)bh * (n[1] + 1) * sizeof(int32_t));
        int32_t *col = malloc((size_t)bh * n[1] * kl[1] * sizeof(int32_t));
        const int bad = oracle_transpose(bh, n[1], kl[1], n[1], idx, ptr, col);
        double sum = 0.0;
        for (int64_t i = 0; i < tok; ++i)
            sum += o[i] + dq[i] + dk[i] + dv[i];
        printf("shape %u: bh %d N %d B %d L %d K %d Le %d drop %d: sum %.6f, transpose out of range %d\n",
               si, bh, N, B, L, K, Le, drop, sum, bad);
        free(q); free(k); free(v); free(dout); free(pq); free(pk); free(pv); free(idx);
        free(gap); free(o); free(lse); free(dq); free(dk); free(dv); free(ptr); free(col);
    }
    printf("done\n");
    return 0;
}
