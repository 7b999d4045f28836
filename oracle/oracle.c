/*
 * fp64 CPU oracle for tile-masked (block-sparse) attention over a T x H x W
 * video token grid.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU library is checked against.  Only the tests, the
 * package smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never does.  It shares no code, header or table with the GPU
 * library.
 *
 * What it computes, and where the pages fix it:
 *
 *  - Masked attention is exact attention restricted to the kept keys.  The
 *    SCOPE review page (abstract) says sparse attention is computed over the
 *    selected original keys and values, and ("If this is right") that
 *    attention uses the original tokens; the 1/sqrt(d) scale is the one in
 *    its proxy logit ("What carries the argument").  So for head h and query
 *    token n with kept key set J = { m : M_h[tile(n), tile(m)] != 0 }:
 *        O[h, n] = sum_{m in J} exp(s q_n.k_m - mu) v_m / sum_{m in J} exp(s q_n.k_m - mu)
 *    with mu the maximum score over J, all in double precision; an empty J
 *    gives O = 0.
 *
 *  - The log-sum-exp of a query row's kept scores,
 *        LSE[h, n] = mu + ln sum_{m in J} exp(s q_n.k_m - mu),
 *    natural log, -infinity for an empty J.  It is the per-row statistic the
 *    AdaSpa page (abstract) caches across denoising steps; with it the
 *    weights of any key are exp(s q_n.k_m - LSE) without another pass.
 *
 *  - Masks are per head and per pair of tiles (Compact Attention page,
 *    abstract: head-specific masks in one tile-aligned family; Fig. 3
 *    caption: precomputed masks are loaded into block-sparse attention
 *    kernels).  Tokens are numbered raster n = (t H + y) W + x and tiles
 *    (tt, th, tw) are numbered raster over the tile grid; a grid that the
 *    tile does not divide gets clipped tiles at the far edges.
 *
 *  - Dual-window masks (Compact Attention page, Fig. 1 caption part (3) and
 *    Fig. 4 caption: two deformable windows per temporal-distance group).
 *    The pages give no formula; the reading used here: a pair of tiles
 *    (a_i, b_i, e_i) -> (a_j, b_j, e_j) is kept when |a_i - a_j| lies in one
 *    of the head's groups [dt_lo, dt_hi] (dt_hi = -1: unbounded) and, for
 *    some window w of that group with both half-extents >= 0,
 *    |b_i - b_j| <= ry_w and |e_i - e_j| <= rx_w.
 *
 *  - The tile-major layout is the slot map of a "tile-aligned" mask family:
 *    tile tau owns slots [tau B, (tau + 1) B) with B = tt th tw; its real
 *    tokens fill the first c_tau slots in raster order over the clipped tile
 *    and the rest are empty (-1).
 *
 *  - The compiled index lists: per row r = h nT + i, the kept key tiles in
 *    ascending order; row offsets by exclusive sum of the row lengths; a work
 *    order of rows by decreasing length, ties by row id.
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

typedef struct {
    int64_t T, H, W;    /* token grid */
    int64_t tt, th, tw; /* tile shape */
} oracle_grid;

typedef struct {
    int32_t dt_lo, dt_hi;
    int32_t ry[2];
    int32_t rx[2];
} oracle_group;

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

/* Number of tiles of the grid. */
int64_t oracle_num_tiles(const oracle_grid *g)
{
    return cdiv(g->T, g->tt) * cdiv(g->H, g->th) * cdiv(g->W, g->tw);
}

/* Tile id of token n. */
static int64_t tile_of_token(const oracle_grid *g, int64_t n)
{
    int64_t t = n / (g->H * g->W);
    int64_t y = (n / g->W) % g->H;
    int64_t x = n % g->W;
    int64_t ny = cdiv(g->H, g->th), nx = cdiv(g->W, g->tw);
    return ((t / g->tt) * ny + y / g->th) * nx + x / g->tw;
}

/* Real token count of every tile: counts[nT]. */
void oracle_tile_counts(const oracle_grid *g, int64_t *counts)
{
    int64_t nT = oracle_num_tiles(g);
    int64_t N = g->T * g->H * g->W;
    memset(counts, 0, sizeof(int64_t) * (size_t)nT);
    for (int64_t n = 0; n < N; ++n)
        counts[tile_of_token(g, n)] += 1;
}

/*
 * Slot maps of the tile-major layout.  perm[nT * B]: token held by each slot,
 * or -1 for an empty slot.  pos[N]: slot of each token.
 */
void oracle_perm(const oracle_grid *g, int64_t *perm, int64_t *pos)
{
    int64_t nT = oracle_num_tiles(g);
    int64_t B = g->tt * g->th * g->tw;
    int64_t N = g->T * g->H * g->W;
    for (int64_t p = 0; p < nT * B; ++p)
        perm[p] = -1;
    for (int64_t n = 0; n < N; ++n) {
        int64_t t = n / (g->H * g->W);
        int64_t y = (n / g->W) % g->H;
        int64_t x = n % g->W;
        int64_t a = t / g->tt, b = y / g->th, e = x / g->tw;
        /* clipped extents of this token's tile */
        int64_t ey = min64(g->th, g->H - b * g->th);
        int64_t ex = min64(g->tw, g->W - e * g->tw);
        int64_t rank = ((t - a * g->tt) * ey + (y - b * g->th)) * ex + (x - e * g->tw);
        int64_t slot = tile_of_token(g, n) * B + rank;
        perm[slot] = n;
        pos[n] = slot;
    }
}

/*
 * Hilbert-curve token order (DFSAttn page, abstract: tokens are reordered
 * along a Hilbert curve so that runs of consecutive tokens are compact in
 * space, which keeps block-sparse execution efficient at a finer grain).
 * The page gives no construction; the curve used is the 3D Hilbert curve of
 * J. Skilling, "Programming the Hilbert curve", AIP Conf. Proc. 707 (2004),
 * over the smallest cube of side 2^k that holds the grid, axes (t, y, x),
 * its 3k index bits read level by level from the top with t's bit first.
 *
 * The oracle walks the curve from index to point.  Skilling's point-to-index
 * map ends by reading the interleaved coordinate bits (after its per-level
 * exchanges) as a Gray code and decoding it, so from an index h the
 * interleaved bits are the Gray code h ^ (h >> 1), dealt back to the axes.
 * The per-level steps are then undone in reverse: each exchange or
 * reflection of the bits below level Q is its own inverse, and the bit it
 * tests (bit Q of an axis) is not changed by the steps of level Q and
 * below, so the steps are replayed from the lowest level up, within a level
 * from the last axis to the first.  The order of a grid lists the cube's
 * points in index order, skipping those outside the grid; runs of B
 * consecutive ranks then take the place of tiles, so the layout is the tile
 * layout of a 1 x 1 x N grid in rank order.
 */
static int cube_order(int64_t T, int64_t H, int64_t W)
{
    int64_t m = T > H ? T : H;
    if (W > m)
        m = W;
    int k = 0;
    while (((int64_t)1 << k) < m)
        ++k;
    return k;
}

/* The point (t, y, x) of index h on the curve over the 2^k cube. */
void oracle_hilbert_point(int k, uint64_t h, int64_t *t, int64_t *y, int64_t *x)
{
    const uint64_t gray = h ^ (h >> 1);
    uint64_t X[3] = {0, 0, 0};
    /* Bit 3 b + 2 - i of the index belongs to axis i at level b. */
    for (int b = 0; b < k; ++b)
        for (int i = 0; i < 3; ++i)
            X[i] |= ((gray >> (3 * b + 2 - i)) & 1) << b;
    for (int b = 1; b < k; ++b) {
        const uint64_t Q = (uint64_t)1 << b, low = Q - 1;
        for (int i = 2; i >= 0; --i) {
            if (X[i] & Q) {
                X[0] ^= low; /* reflection of axis 0's lower bits */
            } else {
                uint64_t d = (X[0] ^ X[i]) & low; /* exchange with axis i */
                X[0] ^= d;
                X[i] ^= d;
            }
        }
    }
    *t = (int64_t)X[0];
    *y = (int64_t)X[1];
    *x = (int64_t)X[2];
}

/* seq[r] = raster token of Hilbert rank r, for r in [0, T H W). */
void oracle_hilbert_order(int64_t T, int64_t H, int64_t W, int64_t *seq)
{
    const int k = cube_order(T, H, W);
    const uint64_t cells = (uint64_t)1 << (3 * k);
    int64_t r = 0;
    for (uint64_t h = 0; h < cells; ++h) {
        int64_t t, y, x;
        oracle_hilbert_point(k, h, &t, &y, &x);
        if (t < T && y < H && x < W)
            seq[r++] = (t * H + y) * W + x;
    }
}

/*
 * Evaluate dual-window specs into a dense tile mask M[heads][nT][nT].
 * groups holds the groups of head 0, then head 1, ...; groups_per_head[h]
 * of them per head.
 */
void oracle_mask_from_windows(const oracle_grid *g, int64_t heads, const oracle_group *groups,
                              const int32_t *groups_per_head, uint8_t *M)
{
    int64_t ny = cdiv(g->H, g->th), nx = cdiv(g->W, g->tw);
    int64_t nT = oracle_num_tiles(g);
    int64_t first = 0;
    for (int64_t h = 0; h < heads; ++h) {
        const oracle_group *gh = groups + first;
        int32_t ng = groups_per_head[h];
        first += ng;
        for (int64_t i = 0; i < nT; ++i) {
            int64_t ai = i / (ny * nx), bi = (i / nx) % ny, ei = i % nx;
            for (int64_t j = 0; j < nT; ++j) {
                int64_t aj = j / (ny * nx), bj = (j / nx) % ny, ej = j % nx;
                int64_t dt = llabs(ai - aj), dy = llabs(bi - bj), dx = llabs(ei - ej);
                uint8_t keep = 0;
                for (int32_t k = 0; k < ng && !keep; ++k) {
                    const oracle_group *G = &gh[k];
                    if (dt < G->dt_lo || (G->dt_hi >= 0 && dt > G->dt_hi))
                        continue;
                    for (int w = 0; w < 2; ++w) {
                        if (G->ry[w] < 0 || G->rx[w] < 0)
                            continue;
                        if (dy <= G->ry[w] && dx <= G->rx[w])
                            keep = 1;
                    }
                }
                M[(h * nT + i) * nT + j] = keep;
            }
        }
    }
}

typedef struct {
    int64_t len;
    int64_t row;
} len_row;

static int cmp_len_row(const void *pa, const void *pb)
{
    const len_row *a = (const len_row *)pa, *b = (const len_row *)pb;
    if (a->len != b->len)
        return a->len > b->len ? -1 : 1; /* longer first */
    return a->row < b->row ? -1 : (a->row > b->row ? 1 : 0);
}

/*
 * Index lists of a dense mask M[heads][nT][nT] (nonzero = keep).
 * row_ptr[heads * nT + 1]; cols[nnz] (may be NULL to only count);
 * order[heads * nT] (may be NULL).  Returns nnz.
 */
int64_t oracle_csr(const uint8_t *M, int64_t heads, int64_t nT, int64_t *row_ptr, int64_t *cols,
                   int64_t *order)
{
    int64_t R = heads * nT;
    int64_t nnz = 0;
    for (int64_t r = 0; r < R; ++r) {
        row_ptr[r] = nnz;
        for (int64_t j = 0; j < nT; ++j) {
            if (M[r * nT + j]) {
                if (cols)
                    cols[nnz] = j;
                ++nnz;
            }
        }
    }
    row_ptr[R] = nnz;
    if (order) {
        len_row *lr = (len_row *)malloc(sizeof(len_row) * (size_t)(R > 0 ? R : 1));
        for (int64_t r = 0; r < R; ++r) {
            lr[r].len = row_ptr[r + 1] - row_ptr[r];
            lr[r].row = r;
        }
        qsort(lr, (size_t)R, sizeof(len_row), cmp_len_row);
        for (int64_t r = 0; r < R; ++r)
            order[r] = lr[r].row;
        free(lr);
    }
    return nnz;
}

/* Element idx of an input tensor as a double: dtype 0 = fp32, 1 = bf16 bits. */
static double load_elem(const void *p, int dtype, int64_t idx)
{
    if (dtype == 0)
        return (double)((const float *)p)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t *)p)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * Masked softmax attention for selected query rows.
 *   q, k, v: [heads][N][d] of the given dtype.
 *   M: dense tile mask [heads][nT][nT].
 *   rows[count]: flattened query ids h * N + n.
 *   out[count][d]: fp64 outputs.
 *   lse[count]: log-sum-exp of each row's kept scores, or NULL.
 *   scale: score scale s (the caller passes 1/sqrt(d) by default).
 */
void oracle_attention_rows(const oracle_grid *g, int64_t heads, int64_t d, int dtype, const void *q,
                           const void *k, const void *v, const uint8_t *M, double scale,
                           const int64_t *rows, int64_t count, double *out, double *lse,
                           int nthreads)
{
    int64_t N = g->T * g->H * g->W;
    int64_t nT = oracle_num_tiles(g);
    int64_t *tile = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
    for (int64_t n = 0; n < N; ++n)
        tile[n] = tile_of_token(g, n);
    (void)heads;

    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel
    {
        double *score = (double *)malloc(sizeof(double) * (size_t)N);
        double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 4)
        for (int64_t c = 0; c < count; ++c) {
            int64_t h = rows[c] / N, n = rows[c] % N;
            const uint8_t *Mrow = M + (h * nT + tile[n]) * nT;
            for (int64_t e = 0; e < d; ++e)
                qrow[e] = load_elem(q, dtype, (h * N + n) * d + e);
            /* scores over the kept keys and their maximum */
            double mu = -INFINITY;
            int any = 0;
            for (int64_t m = 0; m < N; ++m) {
                if (!Mrow[tile[m]])
                    continue;
                double dot = 0.0;
                for (int64_t e = 0; e < d; ++e)
                    dot += qrow[e] * load_elem(k, dtype, (h * N + m) * d + e);
                score[m] = scale * dot;
                if (score[m] > mu)
                    mu = score[m];
                any = 1;
            }
            for (int64_t e = 0; e < d; ++e)
                acc[e] = 0.0;
            if (lse)
                lse[c] = -INFINITY;
            if (any) {
                double den = 0.0;
                for (int64_t m = 0; m < N; ++m) {
                    if (!Mrow[tile[m]])
                        continue;
                    double w = exp(score[m] - mu);
                    den += w;
                    for (int64_t e = 0; e < d; ++e)
                        acc[e] += w * load_elem(v, dtype, (h * N + m) * d + e);
                }
                for (int64_t e = 0; e < d; ++e)
                    acc[e] /= den;
                if (lse)
                    lse[c] = mu + log(den);
            }
            memcpy(out + c * d, acc, sizeof(double) * (size_t)d);
        }
        free(score);
        free(qrow);
        free(acc);
    }
    free(tile);
}

/*
 * Attention probabilities of one head, for small grids: P[N][N] with
 * P[n][m] the weight query n gives key m (zero for keys it does not keep).
 */
void oracle_probabilities(const oracle_grid *g, int64_t d, int dtype, const void *q, const void *k,
                          const uint8_t *Mh, double scale, double *P)
{
    int64_t N = g->T * g->H * g->W;
    int64_t nT = oracle_num_tiles(g);
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *Mrow = Mh + tile_of_token(g, n) * nT;
        double mu = -INFINITY;
        for (int64_t m = 0; m < N; ++m) {
            P[n * N + m] = 0.0;
            if (!Mrow[tile_of_token(g, m)])
                continue;
            double dot = 0.0;
            for (int64_t e = 0; e < d; ++e)
                dot += load_elem(q, dtype, n * d + e) * load_elem(k, dtype, m * d + e);
            P[n * N + m] = scale * dot;
            if (P[n * N + m] > mu)
                mu = P[n * N + m];
        }
        double den = 0.0;
        for (int64_t m = 0; m < N; ++m) {
            if (!Mrow[tile_of_token(g, m)])
                continue;
            P[n * N + m] = exp(P[n * N + m] - mu);
            den += P[n * N + m];
        }
        for (int64_t m = 0; m < N; ++m)
            if (Mrow[tile_of_token(g, m)])
                P[n * N + m] /= den;
    }
}

/*
 * Tile selection by block-level proxy scores (SCOPE review page: the
 * abstract names masks built from block-level proxy scores, "The reading"
 * a per-head Top-k count, "What carries the argument" the 1/sqrt(d) scale of
 * a proxy logit; AdaSpa page, abstract: a blockified pattern).  The reading
 * used here, the plainest block-level proxy: the score of tile pair (i, j)
 * is scale * qbar_i . kbar_j with qbar, kbar the means of the tiles' real
 * tokens, and row i of head h keeps the k_h tiles with the largest score,
 * ties to the lower j.
 */

/* Mean of each tile's real tokens: x [N][d] of the given dtype -> out [nT][d]. */
void oracle_tile_means(const oracle_grid *g, int64_t d, int dtype, const void *x, double *out)
{
    int64_t N = g->T * g->H * g->W;
    int64_t nT = oracle_num_tiles(g);
    int64_t *cnt = calloc((size_t)nT, sizeof *cnt);
    memset(out, 0, (size_t)(nT * d) * sizeof *out);
    for (int64_t n = 0; n < N; ++n) {
        int64_t t = tile_of_token(g, n);
        cnt[t] += 1;
        for (int64_t e = 0; e < d; ++e)
            out[t * d + e] += load_elem(x, dtype, n * d + e);
    }
    for (int64_t t = 0; t < nT; ++t)
        for (int64_t e = 0; e < d; ++e)
            out[t * d + e] = cnt[t] ? out[t * d + e] / (double)cnt[t] : 0.0;
    free(cnt);
}

typedef struct {
    double score;
    int64_t j;
} scored_tile;

/* Larger score first, then lower tile id. */
static int cmp_score(const void *pa, const void *pb)
{
    const scored_tile *a = pa, *b = pb;
    if (a->score != b->score)
        return a->score > b->score ? -1 : 1;
    return (a->j > b->j) - (a->j < b->j);
}

/*
 * q, k: [heads][N][d]; kh[heads] in 0..nT; M: [heads][nT][nT] (0/1) out.
 */
void oracle_select_topk(const oracle_grid *g, int64_t heads, int64_t d, int dtype, const void *q,
                        const void *k, const int64_t *kh, double scale, uint8_t *M, int nthreads)
{
    int64_t N = g->T * g->H * g->W;
    int64_t nT = oracle_num_tiles(g);
    size_t esz = dtype == 0 ? 4 : 2;
    double *qb = malloc((size_t)(nT * d) * sizeof *qb);
    double *kb = malloc((size_t)(nT * d) * sizeof *kb);
    for (int64_t h = 0; h < heads; ++h) {
        oracle_tile_means(g, d, dtype, (const char *)q + (size_t)(h * N * d) * esz, qb);
        oracle_tile_means(g, d, dtype, (const char *)k + (size_t)(h * N * d) * esz, kb);
#pragma omp parallel for schedule(dynamic, 8) num_threads(nthreads)
        for (int64_t i = 0; i < nT; ++i) {
            scored_tile *row = malloc((size_t)nT * sizeof *row);
            for (int64_t j = 0; j < nT; ++j) {
                double dot = 0.0;
                for (int64_t e = 0; e < d; ++e)
                    dot += qb[i * d + e] * kb[j * d + e];
                row[j].score = scale * dot;
                row[j].j = j;
            }
            qsort(row, (size_t)nT, sizeof *row, cmp_score);
            uint8_t *Mrow = M + (h * nT + i) * nT;
            memset(Mrow, 0, (size_t)nT);
            for (int64_t r = 0; r < kh[h] && r < nT; ++r)
                Mrow[row[r].j] = 1;
            free(row);
        }
    }
    free(qb);
    free(kb);
}

/*
 * Reference attention mass per tile pair, the quantity the offline mask
 * search works on (Compact Attention page, Fig. 1 caption: reference
 * attention mass of query-key regions; Fig. 4 caption: the search keeps the
 * regions that hold most of each head's attention mass).  The reference is
 * full attention: for query token n of head h,
 *     p(n, m) = exp(s q_n.k_m - mu_n) / sum_{m' < N} exp(s q_n.k_m' - mu_n)
 * over all N keys, and for query tile i, key tile j
 *     A[h][i][j] = (1 / c_i) sum_{n in tile i} sum_{m in tile j} p(n, m),
 * the mean over the tile's real queries of the mass they give tile j.
 * Only the query tiles listed in qtiles[count] (flattened h nT + i) are
 * evaluated: out[count][nT].
 */
void oracle_tile_mass(const oracle_grid *g, int64_t heads, int64_t d, int dtype, const void *q,
                      const void *k, double scale, const int64_t *qtiles, int64_t count, double *out,
                      int nthreads)
{
    int64_t N = g->T * g->H * g->W;
    int64_t nT = oracle_num_tiles(g);
    int64_t *tile = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
    int64_t *cnt = (int64_t *)calloc((size_t)nT, sizeof(int64_t));
    for (int64_t n = 0; n < N; ++n) {
        tile[n] = tile_of_token(g, n);
        cnt[tile[n]] += 1;
    }
    (void)heads;
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel
    {
        double *score = (double *)malloc(sizeof(double) * (size_t)N);
        double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t c = 0; c < count; ++c) {
            int64_t h = qtiles[c] / nT, i = qtiles[c] % nT;
            double *row = out + c * nT;
            for (int64_t j = 0; j < nT; ++j)
                row[j] = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                if (tile[n] != i)
                    continue;
                for (int64_t e = 0; e < d; ++e)
                    qrow[e] = load_elem(q, dtype, (h * N + n) * d + e);
                double mu = -INFINITY;
                for (int64_t m = 0; m < N; ++m) {
                    double dot = 0.0;
                    for (int64_t e = 0; e < d; ++e)
                        dot += qrow[e] * load_elem(k, dtype, (h * N + m) * d + e);
                    score[m] = scale * dot;
                    if (score[m] > mu)
                        mu = score[m];
                }
                double den = 0.0;
                for (int64_t m = 0; m < N; ++m)
                    den += exp(score[m] - mu);
                for (int64_t m = 0; m < N; ++m)
                    row[tile[m]] += exp(score[m] - mu) / den / (double)cnt[i];
            }
        }
        free(score);
        free(qrow);
    }
    free(tile);
    free(cnt);
}
