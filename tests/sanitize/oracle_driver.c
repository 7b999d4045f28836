/* The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (built
 * and run by tests/test_sanitizers.py on the CPU): every exported function on
 * small grids with clipped tiles, empty and full masks, both dtypes and the
 * Hilbert order, with a few invariants checked on the way.  The oracle is
 * test infrastructure; this is a check of it, not a second oracle. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t T, H, W;
    int64_t tt, th, tw;
} oracle_grid;

typedef struct {
    int32_t dt_lo, dt_hi;
    int32_t ry[2];
    int32_t rx[2];
} oracle_group;

int64_t oracle_num_tiles(const oracle_grid *g);
void oracle_tile_counts(const oracle_grid *g, int64_t *counts);
void oracle_perm(const oracle_grid *g, int64_t *perm, int64_t *pos);
void oracle_hilbert_point(int k, uint64_t h, int64_t *t, int64_t *y, int64_t *x);
void oracle_hilbert_order(int64_t T, int64_t H, int64_t W, int64_t *seq);
void oracle_mask_from_windows(const oracle_grid *g, int64_t heads, const oracle_group *groups,
                              const int32_t *groups_per_head, uint8_t *M);
int64_t oracle_csr(const uint8_t *M, int64_t heads, int64_t nT, int64_t *row_ptr, int64_t *cols, int64_t *order);
void oracle_attention_rows(const oracle_grid *g, int64_t heads, int64_t d, int dtype, const void *q, const void *k,
                           const void *v, const uint8_t *M, double scale, const int64_t *rows, int64_t count,
                           double *out, double *lse, int nthreads);
void oracle_probabilities(const oracle_grid *g, int64_t d, int dtype, const void *q, const void *k,
                          const uint8_t *Mh, double scale, double *P);
void oracle_tile_means(const oracle_grid *g, int64_t d, int dtype, const void *x, double *out);
void oracle_select_topk(const oracle_grid *g, int64_t heads, int64_t d, int dtype, const void *q, const void *k,
                        const int64_t *kh, double scale, uint8_t *M, int nthreads);
void oracle_tile_mass(const oracle_grid *g, int64_t heads, int64_t d, int dtype, const void *q, const void *k,
                      double scale, const int64_t *qtiles, int64_t count, double *out, int nthreads);

static int fails = 0;
#define EXPECT(c)                                                                  \
    do {                                                                           \
        if (!(c)) {                                                                \
            fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #c);         \
            ++fails;                                                               \
        }                                                                          \
    } while (0)

static uint32_t rng_state = 12345u;
static double urand(void)
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return (double)(rng_state >> 8) / 16777216.0;
}

static void run_grid(oracle_grid g, int64_t heads, int64_t d, int dtype)
{
    const int64_t N = g.T * g.H * g.W, nT = oracle_num_tiles(&g), B = g.tt * g.th * g.tw;
    int64_t *counts = malloc(sizeof(int64_t) * (size_t)nT);
    oracle_tile_counts(&g, counts);
    int64_t sum = 0;
    for (int64_t t = 0; t < nT; ++t)
        sum += counts[t];
    EXPECT(sum == N);
    int64_t *perm = malloc(sizeof(int64_t) * (size_t)(nT * B)), *pos = malloc(sizeof(int64_t) * (size_t)N);
    oracle_perm(&g, perm, pos);
    for (int64_t n = 0; n < N; ++n)
        EXPECT(perm[pos[n]] == n);

    const size_t esz = dtype == 0 ? 4 : 2, nel = (size_t)(heads * N * d);
    void *q = malloc(esz * nel), *k = malloc(esz * nel), *v = malloc(esz * nel);
    for (size_t i = 0; i < nel; ++i) {
        float a = (float)(2 * urand() - 1), b = (float)(2 * urand() - 1), c = (float)(2 * urand() - 1);
        if (dtype == 0) {
            ((float *)q)[i] = a;
            ((float *)k)[i] = b;
            ((float *)v)[i] = c;
        } else {
            uint32_t ua, ub, uc;
            memcpy(&ua, &a, 4);
            memcpy(&ub, &b, 4);
            memcpy(&uc, &c, 4);
            ((uint16_t *)q)[i] = (uint16_t)(ua >> 16);
            ((uint16_t *)k)[i] = (uint16_t)(ub >> 16);
            ((uint16_t *)v)[i] = (uint16_t)(uc >> 16);
        }
    }
    /* Masks: random, window spec, empty. */
    uint8_t *M = malloc((size_t)(heads * nT * nT));
    for (int64_t i = 0; i < heads * nT * nT; ++i)
        M[i] = urand() < 0.4;
    oracle_group groups[4] = {{0, 0, {1, 0}, {0, 2}}, {1, -1, {0, -1}, {1, -1}},
                              {0, 1, {-1, 0}, {-1, 0}}, {2, -1, {2, 2}, {0, 0}}};
    int32_t *gph = malloc(sizeof(int32_t) * (size_t)heads);
    oracle_group *gall = malloc(sizeof(oracle_group) * (size_t)(2 * heads));
    for (int64_t h = 0; h < heads; ++h) {
        gph[h] = 2;
        gall[2 * h] = groups[(h % 2) * 2];
        gall[2 * h + 1] = groups[(h % 2) * 2 + 1];
    }
    uint8_t *W = malloc((size_t)(heads * nT * nT));
    oracle_mask_from_windows(&g, heads, gall, gph, W);
    for (int64_t i = 0; i < nT; ++i)
        EXPECT(W[i * nT + i] == 1); /* head 0: window 0 of group 0 keeps the own tile */
    int64_t *row_ptr = malloc(sizeof(int64_t) * (size_t)(heads * nT + 1));
    const int64_t nnz = oracle_csr(M, heads, nT, row_ptr, NULL, NULL);
    int64_t *cols = malloc(sizeof(int64_t) * (size_t)(nnz > 0 ? nnz : 1));
    int64_t *order = malloc(sizeof(int64_t) * (size_t)(heads * nT));
    EXPECT(oracle_csr(M, heads, nT, row_ptr, cols, order) == nnz);
    EXPECT(row_ptr[heads * nT] == nnz);

    /* Attention rows (every query of every head) with LSE, the probability
     * matrix of head 0, tile means, selection, tile mass. */
    const int64_t R = heads * N;
    int64_t *rows = malloc(sizeof(int64_t) * (size_t)R);
    for (int64_t r = 0; r < R; ++r)
        rows[r] = r;
    double *out = malloc(sizeof(double) * (size_t)(R * d)), *lse = malloc(sizeof(double) * (size_t)R);
    const double s = 1.0 / sqrt((double)d);
    oracle_attention_rows(&g, heads, d, dtype, q, k, v, M, s, rows, R, out, lse, 2);
    for (int64_t r = 0; r < R * d; ++r)
        EXPECT(isfinite(out[r]));
    uint8_t *E = calloc((size_t)(heads * nT * nT), 1);
    oracle_attention_rows(&g, heads, d, dtype, q, k, v, E, s, rows, R, out, lse, 1);
    for (int64_t r = 0; r < R; ++r)
        EXPECT(isinf(lse[r]) && lse[r] < 0 && out[r * d] == 0.0);
    double *P = malloc(sizeof(double) * (size_t)(N * N));
    oracle_probabilities(&g, d, dtype, q, k, M, s, P);
    for (int64_t n = 0; n < N; ++n) {
        double rs = 0;
        int64_t kept = 0;
        for (int64_t m = 0; m < N; ++m)
            rs += P[n * N + m];
        for (int64_t j = 0; j < nT; ++j)
            kept += M[(pos[n] / B) * nT + j];
        EXPECT(kept == 0 ? rs == 0.0 : fabs(rs - 1.0) < 1e-12);
    }
    double *means = malloc(sizeof(double) * (size_t)(nT * d));
    oracle_tile_means(&g, d, dtype, q, means);
    int64_t *kh = malloc(sizeof(int64_t) * (size_t)heads);
    for (int64_t h = 0; h < heads; ++h)
        kh[h] = h % (nT + 1);
    uint8_t *S = malloc((size_t)(heads * nT * nT));
    oracle_select_topk(&g, heads, d, dtype, q, k, kh, s, S, 2);
    for (int64_t h = 0; h < heads; ++h)
        for (int64_t i = 0; i < nT; ++i) {
            int64_t c = 0;
            for (int64_t j = 0; j < nT; ++j)
                c += S[(h * nT + i) * nT + j];
            EXPECT(c == kh[h]);
        }
    int64_t *qt = malloc(sizeof(int64_t) * (size_t)(heads * nT));
    for (int64_t t = 0; t < heads * nT; ++t)
        qt[t] = t;
    double *mass = malloc(sizeof(double) * (size_t)(heads * nT * nT));
    oracle_tile_mass(&g, heads, d, dtype, q, k, s, qt, heads * nT, mass, 2);
    for (int64_t r = 0; r < heads * nT; ++r) {
        double rs = 0;
        for (int64_t j = 0; j < nT; ++j)
            rs += mass[r * nT + j];
        EXPECT(fabs(rs - 1.0) < 1e-12);
    }
    free(counts); free(perm); free(pos); free(q); free(k); free(v); free(M); free(gph); free(gall); free(W);
    free(row_ptr); free(cols); free(order); free(rows); free(out); free(lse); free(E); free(P); free(means);
    free(kh); free(S); free(qt); free(mass);
}

int main(void)
{
    const oracle_grid grids[] = {{4, 8, 8, 1, 4, 4}, {3, 5, 7, 2, 2, 3}, {2, 9, 10, 1, 8, 16}, {1, 1, 1, 1, 1, 1},
                                 {5, 3, 3, 2, 3, 3}};
    for (size_t i = 0; i < sizeof grids / sizeof grids[0]; ++i) {
        run_grid(grids[i], 2, 8, 0);
        run_grid(grids[i], 3, 16, 1);
    }
    /* Hilbert order: a bijection onto the grid, unit steps on a full cube. */
    const int64_t dims[][3] = {{4, 4, 4}, {3, 5, 7}, {1, 1, 9}, {8, 2, 2}};
    for (size_t i = 0; i < sizeof dims / sizeof dims[0]; ++i) {
        const int64_t T = dims[i][0], H = dims[i][1], W = dims[i][2], N = T * H * W;
        int64_t *seq = malloc(sizeof(int64_t) * (size_t)N);
        char *seen = calloc((size_t)N, 1);
        oracle_hilbert_order(T, H, W, seq);
        for (int64_t r = 0; r < N; ++r) {
            EXPECT(seq[r] >= 0 && seq[r] < N && !seen[seq[r]]);
            if (seq[r] >= 0 && seq[r] < N)
                seen[seq[r]] = 1;
        }
        free(seq);
        free(seen);
    }
    for (uint64_t hh = 0; hh < 512; ++hh) {
        int64_t t, y, x;
        oracle_hilbert_point(3, hh, &t, &y, &x);
        EXPECT(t >= 0 && t < 8 && y >= 0 && y < 8 && x >= 0 && x < 8);
    }
    printf("oracle checks done, %d failure(s)\n", fails);
    return fails ? 1 : 0;
}
