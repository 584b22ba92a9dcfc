/*
 * llsa_oracle.c -- slow, plain fp64 CPU oracle for Log-linear Sparse Attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the HIP library; it is written from the method's description:
 *
 *   "Trainable Log-linear Sparse Attention for Efficient Diffusion
 *    Transformers" (howistudyai.com explainer), section "Building Blocks" and
 *   the walkthrough "Step 1: Hierarchical Compression", "Step 2: Hierarchical
 *   Top-K Selection", "Step 3: Hierarchical KV Enrichment + KV Reweighting",
 *   "Step 4: Efficient Sparse Index Transpose".
 *
 * Every value is a double.  Tensors are C-contiguous:
 *   tokens     x[bh][N][d]                    (bh = batch * heads)
 *   pyramid    level l = 1..L stored one after the other, level l = [bh][N/B^l][d]
 *   index list level l = 1..L stored one after the other, level l = [bh][N/B^l][K_l]
 * with K_L = min(K, N/B^L) and K_l = min(K, K_{l+1} * B) below the top level
 * (a level never keeps more picks than it has candidates).
 *
 * Readings of the pages taken here where they leave a step open:
 *   - "pool" is the arithmetic mean of B consecutive tokens, applied level by
 *     level (Step 1 names mean pooling as the example operator);
 *   - the similarity used for selection is the raw dot product of pooled
 *     vectors (Step 2 says "similarities");
 *   - ties in Top-K go to the lower index; stored rows are ascending;
 *   - the candidates of level-l query i are the B children of each pick of its
 *     parent i/B at level l+1 (Step 2: the picks "expanded to that level");
 *   - coarse tokens for query block i come from levels 2..Le+1, namely the
 *     picks of i's ancestor at that level, each with weight B^l (Step 3);
 *     a coarse pick all of whose level-1 children are already fine picks of
 *     the block is left out when drop_covered != 0;
 *   - weight w multiplies the unnormalised attention weight: logit + ln w;
 *   - the softmax scale multiplies every dot product before the ln w term.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static int64_t ipow64(int64_t base, int e)
{
    int64_t r = 1;
    while (e-- > 0) r *= base;
    return r;
}

/* Number of picks kept at every level, top level first is computed here
 * bottom-up in the array kl[1..L] (kl[0] unused). */
static void level_k(int N, int B, int L, int K, int *kl)
{
    int64_t nL = N / ipow64(B, L);
    kl[L] = (int)(K < nL ? K : nL);
    for (int l = L - 1; l >= 1; --l) {
        int64_t cand = (int64_t)kl[l + 1] * B;
        kl[l] = (int)(K < cand ? K : cand);
    }
}

/* Offset (in elements) of level l (1-based) in a level-major buffer whose
 * level-l part has bh * n_l * width_l elements. */
static int64_t pyr_offset(int bh, int N, int B, int d, int l)
{
    int64_t off = 0;
    for (int j = 1; j < l; ++j) off += (int64_t)bh * (N / ipow64(B, j)) * d;
    return off;
}

static int64_t idx_offset(int bh, int N, int B, const int *kl, int l)
{
    int64_t off = 0;
    for (int j = 1; j < l; ++j) off += (int64_t)bh * (N / ipow64(B, j)) * kl[j];
    return off;
}

/* ------------------------------------------------------------------------ */
/* Step 1, Hierarchical Compression: level l token j is the mean of the B     */
/* level-(l-1) tokens jB .. jB+B-1; level 0 is the input.                     */
/* ------------------------------------------------------------------------ */
void oracle_pool(int bh, int N, int d, int B, int L, const double *x, double *pyr)
{
    const double *prev = x;
    int64_t n_prev = N;
    double *out = pyr;
    for (int l = 1; l <= L; ++l) {
        int64_t n = n_prev / B;
        for (int h = 0; h < bh; ++h)
            for (int64_t j = 0; j < n; ++j)
                for (int c = 0; c < d; ++c) {
                    double s = 0.0;
                    for (int t = 0; t < B; ++t)
                        s += prev[((int64_t)h * n_prev + j * B + t) * d + c];
                    out[((int64_t)h * n + j) * d + c] = s / B;
                }
        prev = out;
        n_prev = n;
        out += (int64_t)bh * n * d;
    }
}

/* ------------------------------------------------------------------------ */
/* Step 2, Hierarchical Top-K Selection, one level.                           */
/* ------------------------------------------------------------------------ */
typedef struct { double s; int32_t c; } cand_t;

/* order: higher score first, lower index first among equal scores */
static int cand_cmp(const void *a, const void *b)
{
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->c > y->c) - (x->c < y->c);
}

static int int_cmp(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/*
 * q, k   : [bh][n][d] pooled queries / keys of this level.
 * parent : NULL at the coarsest level (all n keys are candidates of every
 *          query); otherwise [bh][n/B][kp], the picks of the level above.
 * out    : [bh][n][kout] with kout = min(K, #candidates); rows ascending.
 * relgap : [bh][n]: (s_(kout) - s_(kout+1)) / max(|s_(kout)|, |s_(kout+1)|)
 *          over the sorted scores; 0 for an exact tie, -1 when every
 *          candidate is kept (there is no (kout+1)-th score).
 * Returns kout.
 */
int oracle_select_level(int bh, int n, int d, int B, int K,
                        const double *q, const double *k,
                        const int32_t *parent, int kp,
                        int32_t *out, double *relgap)
{
    int ncand = parent ? kp * B : n;
    int kout = K < ncand ? K : ncand;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t row = 0; row < (int64_t)bh * n; ++row) {
        int h = (int)(row / n);
        int64_t i = row % n;
        cand_t *cs = (cand_t *)malloc(sizeof(cand_t) * ncand);
        int32_t *keep = (int32_t *)malloc(sizeof(int32_t) * (kout > 0 ? kout : 1));
        for (int m = 0; m < ncand; ++m) {
            int32_t c;
            if (parent) {
                const int32_t *pr = parent + ((int64_t)h * (n / B) + i / B) * kp;
                c = pr[m / B] * B + (m % B);
            } else {
                c = m;
            }
            const double *qi = q + ((int64_t)h * n + i) * d;
            const double *kc = k + ((int64_t)h * n + c) * d;
            double s = 0.0;
            for (int e = 0; e < d; ++e) s += qi[e] * kc[e];
            cs[m].s = s;
            cs[m].c = c;
        }
        qsort(cs, ncand, sizeof(cand_t), cand_cmp);
        for (int m = 0; m < kout; ++m) keep[m] = cs[m].c;
        qsort(keep, kout, sizeof(int32_t), int_cmp);
        memcpy(out + row * kout, keep, sizeof(int32_t) * kout);
        if (relgap) {
            if (kout >= ncand) {
                relgap[row] = -1.0;
            } else {
                double a = cs[kout - 1].s, b = cs[kout].s;
                double m = fabs(a) > fabs(b) ? fabs(a) : fabs(b);
                relgap[row] = (m > 0.0) ? (a - b) / m : 0.0;
            }
        }
        free(cs);
        free(keep);
    }
    return kout;
}

/* All levels, coarse to fine (Step 2): level L densely, then every finer
 * level from the picks of the level above.  idx / relgap are level-major
 * (levels 1..L); relgap level l is [bh][n_l]. */
void oracle_select(int bh, int N, int d, int B, int L, int K,
                   const double *pyr_q, const double *pyr_k,
                   int32_t *idx, double *relgap)
{
    int kl[64];
    level_k(N, B, L, K, kl);
    for (int l = L; l >= 1; --l) {
        int n = (int)(N / ipow64(B, l));
        const double *ql = pyr_q + pyr_offset(bh, N, B, d, l);
        const double *kk = pyr_k + pyr_offset(bh, N, B, d, l);
        int32_t *o = idx + idx_offset(bh, N, B, kl, l);
        const int32_t *par = (l == L) ? NULL : idx + idx_offset(bh, N, B, kl, l + 1);
        int64_t goff = 0;
        for (int j = 1; j < l; ++j) goff += (int64_t)bh * (N / ipow64(B, j));
        oracle_select_level(bh, n, d, B, K, ql, kk, par, (l == L) ? 0 : kl[l + 1],
                            o, relgap ? relgap + goff : NULL);
    }
}

/* ------------------------------------------------------------------------ */
/* Step 3, Hierarchical KV Enrichment + KV Reweighting.                       */
/* The attended set of query block i: every token of every fine block picked */
/* in I^(1)[i] with weight 1, then for l = 2..Le+1 the picks c of the        */
/* block's level-l ancestor a = i / B^(l-1), as pooled tokens K^(l)[c],      */
/* V^(l)[c] with weight B^l (unless all of c's level-1 children are fine     */
/* picks and drop_covered is set).                                            */
/* ------------------------------------------------------------------------ */
typedef struct {
    const double *k;   /* key vector   */
    const double *v;   /* value vector */
    double logw;       /* ln weight    */
    int level;         /* 0 = token, l >= 2 pooled level */
    int64_t pos;       /* token index (level 0) or pooled index at its level */
} kv_t;

/* Fills kv[] for query block i of head h; returns the number of entries. */
static int build_kv(int h, int64_t i, int N, int d, int B, int L, const int *kl, int Le,
                    int drop_covered, const double *k, const double *v,
                    const double *pyr_k, const double *pyr_v, const int32_t *idx,
                    int bh, kv_t *kv)
{
    int cnt = 0;
    int64_t n1 = N / B;
    const int32_t *fine = idx + idx_offset(bh, N, B, kl, 1) + ((int64_t)h * n1 + i) * kl[1];
    for (int m = 0; m < kl[1]; ++m)
        for (int t = 0; t < B; ++t) {
            int64_t u = (int64_t)fine[m] * B + t;
            kv[cnt].k = k + ((int64_t)h * N + u) * d;
            kv[cnt].v = v + ((int64_t)h * N + u) * d;
            kv[cnt].logw = 0.0;
            kv[cnt].level = 0;
            kv[cnt].pos = u;
            ++cnt;
        }
    for (int l = 2; l <= Le + 1 && l <= L; ++l) {
        int64_t nl = N / ipow64(B, l);
        int64_t span = ipow64(B, l - 1);       /* level-1 blocks under one level-l token */
        int64_t a = i / span;                  /* ancestor of block i at level l */
        const int32_t *picks = idx + idx_offset(bh, N, B, kl, l) + ((int64_t)h * nl + a) * kl[l];
        for (int m = 0; m < kl[l]; ++m) {
            int64_t c = picks[m];
            if (drop_covered) {
                int64_t cov = 0;
                for (int f = 0; f < kl[1]; ++f)
                    if (fine[f] / span == c) ++cov;
                if (cov == span) continue;
            }
            int64_t off = pyr_offset(bh, N, B, d, l) + ((int64_t)h * nl + c) * d;
            kv[cnt].k = pyr_k + off;
            kv[cnt].v = pyr_v + off;
            kv[cnt].logw = log((double)ipow64(B, l));
            kv[cnt].level = l;
            kv[cnt].pos = c;
            ++cnt;
        }
    }
    return cnt;
}

static int kv_capacity(int B, int L, const int *kl, int Le)
{
    int cap = kl[1] * B;
    for (int l = 2; l <= Le + 1 && l <= L; ++l) cap += kl[l];
    return cap;
}

/* o[bh][N][d], lse[bh][N] (natural log). */
void oracle_attn_fwd(int bh, int N, int d, int B, int L, int K, int Le, double scale,
                     int drop_covered,
                     const double *q, const double *k, const double *v,
                     const double *pyr_k, const double *pyr_v, const int32_t *idx,
                     double *o, double *lse)
{
    int kl[64];
    level_k(N, B, L, K, kl);
    int64_t n1 = N / B;
    int cap = kv_capacity(B, L, kl, Le);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t blk = 0; blk < (int64_t)bh * n1; ++blk) {
        int h = (int)(blk / n1);
        int64_t i = blk % n1;
        kv_t *kv = (kv_t *)malloc(sizeof(kv_t) * cap);
        double *z = (double *)malloc(sizeof(double) * cap);
        int cnt = build_kv(h, i, N, d, B, L, kl, Le, drop_covered, k, v, pyr_k, pyr_v, idx, bh, kv);
        for (int t = 0; t < B; ++t) {
            int64_t tok = i * B + t;
            const double *qt = q + ((int64_t)h * N + tok) * d;
            double zmax = -INFINITY;
            for (int j = 0; j < cnt; ++j) {
                double s = 0.0;
                for (int e = 0; e < d; ++e) s += qt[e] * kv[j].k[e];
                z[j] = scale * s + kv[j].logw;
                if (z[j] > zmax) zmax = z[j];
            }
            double sum = 0.0;
            for (int j = 0; j < cnt; ++j) sum += exp(z[j] - zmax);
            double l_t = zmax + log(sum);
            double *ot = o + ((int64_t)h * N + tok) * d;
            for (int e = 0; e < d; ++e) ot[e] = 0.0;
            for (int j = 0; j < cnt; ++j) {
                double p = exp(z[j] - l_t);
                for (int e = 0; e < d; ++e) ot[e] += p * kv[j].v[e];
            }
            lse[(int64_t)h * N + tok] = l_t;
        }
        free(kv);
        free(z);
    }
}

/*
 * Gradient of the scalar <O, dO> with respect to Q, K, V for fixed picks
 * (Top-K has no gradient, pooled Q only feeds the picks).  Written query by
 * query with plain accumulation; pooled-token gradients are gathered per
 * level and pushed back through the mean: each of the B^l tokens under a
 * level-l token receives 1/B^l of its gradient.
 */
void oracle_attn_bwd(int bh, int N, int d, int B, int L, int K, int Le, double scale,
                     int drop_covered,
                     const double *q, const double *k, const double *v,
                     const double *pyr_k, const double *pyr_v, const int32_t *idx,
                     const double *dout, double *dq, double *dk, double *dv)
{
    int kl[64];
    level_k(N, B, L, K, kl);
    int64_t n1 = N / B;
    int cap = kv_capacity(B, L, kl, Le);
    int64_t pyr_total = pyr_offset(bh, N, B, d, L + 1);
    memset(dq, 0, sizeof(double) * (size_t)bh * N * d);
    memset(dk, 0, sizeof(double) * (size_t)bh * N * d);
    memset(dv, 0, sizeof(double) * (size_t)bh * N * d);
    double *dpk = (double *)calloc((size_t)pyr_total, sizeof(double));
    double *dpv = (double *)calloc((size_t)pyr_total, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < bh; ++h) {
        kv_t *kv = (kv_t *)malloc(sizeof(kv_t) * cap);
        double *z = (double *)malloc(sizeof(double) * cap);
        double *p = (double *)malloc(sizeof(double) * cap);
        double *ot = (double *)malloc(sizeof(double) * d);
        for (int64_t i = 0; i < n1; ++i) {
            int cnt = build_kv(h, i, N, d, B, L, kl, Le, drop_covered, k, v, pyr_k, pyr_v, idx, bh, kv);
            for (int t = 0; t < B; ++t) {
                int64_t tok = i * B + t;
                const double *qt = q + ((int64_t)h * N + tok) * d;
                const double *gt = dout + ((int64_t)h * N + tok) * d;
                /* forward recomputation */
                double zmax = -INFINITY;
                for (int j = 0; j < cnt; ++j) {
                    double s = 0.0;
                    for (int e = 0; e < d; ++e) s += qt[e] * kv[j].k[e];
                    z[j] = scale * s + kv[j].logw;
                    if (z[j] > zmax) zmax = z[j];
                }
                double sum = 0.0;
                for (int j = 0; j < cnt; ++j) sum += exp(z[j] - zmax);
                double l_t = zmax + log(sum);
                for (int e = 0; e < d; ++e) ot[e] = 0.0;
                for (int j = 0; j < cnt; ++j) {
                    p[j] = exp(z[j] - l_t);
                    for (int e = 0; e < d; ++e) ot[e] += p[j] * kv[j].v[e];
                }
                /* D_t = dO_t . O_t */
                double Dt = 0.0;
                for (int e = 0; e < d; ++e) Dt += gt[e] * ot[e];
                double *dqt = dq + ((int64_t)h * N + tok) * d;
                for (int j = 0; j < cnt; ++j) {
                    double dp = 0.0;
                    for (int e = 0; e < d; ++e) dp += gt[e] * kv[j].v[e];
                    double ds = p[j] * (dp - Dt);
                    double *gk, *gv;
                    if (kv[j].level == 0) {
                        gk = dk + ((int64_t)h * N + kv[j].pos) * d;
                        gv = dv + ((int64_t)h * N + kv[j].pos) * d;
                    } else {
                        int l = kv[j].level;
                        int64_t nl = N / ipow64(B, l);
                        int64_t off = pyr_offset(bh, N, B, d, l) + ((int64_t)h * nl + kv[j].pos) * d;
                        gk = dpk + off;
                        gv = dpv + off;
                    }
                    for (int e = 0; e < d; ++e) {
                        dqt[e] += scale * ds * kv[j].k[e];
                        gk[e] += scale * ds * qt[e];
                        gv[e] += p[j] * gt[e];
                    }
                }
            }
        }
        /* pooled-token gradients back to tokens: mean adjoint */
        for (int l = 2; l <= L; ++l) {
            int64_t nl = N / ipow64(B, l);
            int64_t span = ipow64(B, l);
            int64_t off = pyr_offset(bh, N, B, d, l) + (int64_t)h * nl * d;
            for (int64_t u = 0; u < N; ++u)
                for (int e = 0; e < d; ++e) {
                    dk[((int64_t)h * N + u) * d + e] += dpk[off + (u / span) * d + e] / (double)span;
                    dv[((int64_t)h * N + u) * d + e] += dpv[off + (u / span) * d + e] / (double)span;
                }
        }
        free(kv);
        free(z);
        free(p);
        free(ot);
    }
    free(dpk);
    free(dpv);
}

/* ------------------------------------------------------------------------ */
/* Step 4, sparse index transpose: query-major picks to key-major lists.     */
/* Count the picks of every column, take the exclusive prefix sum as the     */
/* start of each column's segment, then walk the rows in ascending order and */
/* append each row to the segments of the columns it picked.                 */
/* idx [nb][rows][k] -> ptr [nb][cols+1], col [nb][rows*k].                  */
/* Returns 0, or -1 when an index is outside [0, cols).                      */
/* ------------------------------------------------------------------------ */
int oracle_transpose(int nb, int rows, int k, int cols, const int32_t *idx,
                     int32_t *ptr, int32_t *col)
{
    int bad = 0;
    int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)(cols > 0 ? cols : 1));
    for (int b = 0; b < nb; ++b) {
        const int32_t *I = idx + (int64_t)b * rows * k;
        int32_t *P = ptr + (int64_t)b * (cols + 1);
        int32_t *C = col + (int64_t)b * rows * k;
        for (int c = 0; c <= cols; ++c) P[c] = 0;
        for (int64_t e = 0; e < (int64_t)rows * k; ++e) {
            if (I[e] < 0 || I[e] >= cols) { bad = 1; continue; }
            P[I[e] + 1] += 1;
        }
        for (int c = 0; c < cols; ++c) P[c + 1] += P[c];
        for (int c = 0; c < cols; ++c) fill[c] = 0;
        for (int r = 0; r < rows; ++r)
            for (int m = 0; m < k; ++m) {
                int32_t c = I[(int64_t)r * k + m];
                if (c < 0 || c >= cols) continue;
                C[P[c] + fill[c]] = r;
                fill[c] += 1;
            }
    }
    free(fill);
    return bad ? -1 : 0;
}
