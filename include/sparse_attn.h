/*
 * sparse_attn.h - block-sparse (tile-masked) attention forward over a 3D
 * video token grid, for AMD Instinct MI355X (gfx950).
 *
 * The operation.  Video diffusion transformers attend over a latent grid of
 * T x H x W tokens.  The grid is cut into tiles of tt x th x tw tokens and
 * every head h carries its own binary mask M_h over pairs of tiles: query
 * tile i attends to key tile j only when M_h[i, j] is set (Compact Attention
 * page, abstract: head-specific masks in one tile-aligned family; Fig. 1
 * caption: retained query-key regions; Fig. 3 caption: masks are found
 * offline, then compiled once and reused by the block-sparse kernels for
 * several denoising steps in a row).  Inside the kept set the
 * result is exact softmax attention over the original keys and values (SCOPE
 * review page, abstract), with scores scaled by 1/sqrt(head_dim) by default:
 *
 *     O[h, n] = sum_{m kept} softmax_m(s q_n . k_m) v_m,   0 if nothing is kept.
 *
 * Masks come either as a dense tile bitmap or as dual-window specs: per head,
 * temporal-distance groups, each with two rectangular windows of tiles around
 * the query tile (Compact Attention page, Fig. 1 caption part (3); Fig. 4
 * caption).  The pages give no formula for the windows; the reading
 * implemented here is stated at sparse_attn_window_group.
 *
 * Calling pattern (mirrors the pages' offline/online split):
 *     sparse_attn_create        once per shape (host only)
 *     sparse_attn_set_mask      once per mask; compiles it on the GPU
 *     sparse_attn_forward       many times; permute K, V -> attend (Q read and O
 *                               written in place, raster order)
 *     sparse_attn_destroy
 *
 * Conventions shared by every entry point:
 *   - Every call returns a status (SPARSE_ATTN_OK = 0).  All argument checks
 *     finish before anything is enqueued, so a failed call leaves no GPU work
 *     behind.  sparse_attn_last_error() then describes the failure.
 *   - Device pointers are caller-owned HIP device memory (for example torch
 *     tensors), 16-byte aligned.  The library never allocates device memory;
 *     its only device memory of its own is the fixed scratch array of
 *     sparse_attn_forward_noalloc, part of the loaded code object.
 *   - Host arrays a call takes (window specs, per-head k) are read or
 *     staged before the call returns; the caller may reuse them at once.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *     work and return without synchronizing, unless stated otherwise.
 *     Asynchronous faults surface at the caller's next synchronization.
 *   - A handle may not be used by two host threads at once; separate handles
 *     are independent.
 *   - There is no batch dimension: fold batch into heads when grids match.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    SPARSE_ATTN_OK = 0,
    SPARSE_ATTN_INVALID_ARG = 1,         /* null/misaligned/aliased pointer, bad value */
    SPARSE_ATTN_UNSUPPORTED = 2,         /* valid but outside what the library handles */
    SPARSE_ATTN_BAD_MASK = 3,            /* malformed mask description */
    SPARSE_ATTN_WORKSPACE_TOO_SMALL = 4, /* a caller buffer is smaller than required */
    SPARSE_ATTN_NO_MASK = 5,             /* forward/attend before set_mask */
    SPARSE_ATTN_HIP_ERROR = 6,           /* the HIP runtime reported an error */
    SPARSE_ATTN_NO_ORDER = 7             /* Hilbert order without sparse_attn_set_order */
};

/* Element types of Q, K, V and O. */
enum { SPARSE_ATTN_F32 = 0, SPARSE_ATTN_BF16 = 1 };

/* Mask kinds. */
enum { SPARSE_ATTN_MASK_BITMAP = 0, SPARSE_ATTN_MASK_DUAL_WINDOW = 1 };

/* Layouts of a permuted tensor (sparse_attn_permute). */
enum {
    /* [heads][nT * S][head_dim]: slot-major rows, one row per slot (S =
     * sparse_attn_layout_info.slot_stride slots per tile). */
    SPARSE_ATTN_LAYOUT_ROWS = 0,
    /* [heads][nT][head_dim][S]: per tile, one row of S slots per feature
     * (the transposed value tile the MFMA kernel reads). */
    SPARSE_ATTN_LAYOUT_TILE_COLUMNS = 1
};

/* Attention kernels forward may select (sparse_attn_layout_info.kernel). */
enum {
    /* bf16 matrix-core kernels: any tile volume B <= 128, head_dim 64 or
     * 128; every tile takes S = 128 slots (a tile of B < 128 tokens leaves
     * 128 - B of them empty, and that share of the matrix work idle). */
    SPARSE_ATTN_KERNEL_MFMA_BF16 = 0,
    /* vector-ALU kernel, fp32 arithmetic: on request
     * (sparse_attn_config.vector_alu), and for fp32 layouts too large for
     * the fp32 matrix-core kernel; S = B slots per tile. */
    SPARSE_ATTN_KERNEL_GENERIC = 1,
    /* fp32 matrix-core kernel (v_mfma_f32_32x32x2_f32): fp32 inputs, head_dim
     * 64 or 128, S = B slots per tile, while one head's tile-major rows
     * (nT B head_dim 4 bytes) stay below 2^31 bytes. */
    SPARSE_ATTN_KERNEL_MFMA_F32 = 2
};

/*
 * Token orders (sparse_attn_config.order): which tokens form a tile.
 *
 * TILES: tiles are tt x th x tw boxes of the grid, numbered raster over the
 * tile grid (t, then y, then x); edge tiles are clipped.
 *
 * HILBERT: tokens are ranked along a 3D Hilbert curve and tiles are runs of
 * B = tt th tw consecutive ranks (DFSAttn page, abstract: Hilbert-curve
 * token reordering keeps blocks spatially compact at a finer grain than
 * boxes).  The curve is J. Skilling's ("Programming the Hilbert curve",
 * AIP Conf. Proc. 707, 2004) over the smallest cube of side 2^k holding
 * the grid, axes (t, y, x), its index bits read level by level from the
 * top with t's first; cube cells outside the grid are skipped.  Everything
 * that describes tiles then describes a 1 x 1 x N grid of tokens in rank
 * order cut into 1 x 1 x B tiles: nT = ceil(N / B), tile_grid = (1, 1, nT),
 * only the last tile is clipped, and a dual-window group reduces to a band
 * |i - j| <= rx[w] of tiles along the curve.  The rank -> token map lives in
 * a caller-owned device buffer (sparse_attn_order_bytes /
 * sparse_attn_set_order); results do not depend on the order, only which
 * tokens share a tile does.
 */
enum { SPARSE_ATTN_ORDER_TILES = 0, SPARSE_ATTN_ORDER_HILBERT = 1 };

/* Maximum temporal-distance groups per head in a dual-window mask. */
#define SPARSE_ATTN_MAX_GROUPS 8

/*
 * How the matrix-core path splits query tiles between its two kernels
 * (sparse_attn_config.pairing).  The pair kernel runs two neighbouring query
 * tiles per workgroup over the union of their key lists; the row kernel runs
 * one query tile per workgroup.  This is the library's own work split (the
 * pages define only the per-tile mask); results are the same either way.
 *   AUTO    (0): NONE when the layout has at most 1024 pairs over all
 *                heads (too little work to fill the GPU: one-tile work
 *                items, two per compute unit, balance it best), otherwise
 *                OVERLAP.
 *   OVERLAP (1): a pair goes to the pair kernel when the union of its two
 *                lists is at most 7/10 of their total length (and when both
 *                are empty); its tiles go to the row kernel otherwise.
 *   ALL     (2): every pair goes to the pair kernel; no row-kernel launch.
 *   NONE    (3): every tile goes to the row kernel; no pair-kernel launch.
 * The fp32 matrix-core and vector-ALU kernels ignore it (one launch of
 * one kernel serves every query tile).
 */
enum {
    SPARSE_ATTN_PAIRING_AUTO = 0,
    SPARSE_ATTN_PAIRING_OVERLAP = 1,
    SPARSE_ATTN_PAIRING_ALL = 2,
    SPARSE_ATTN_PAIRING_NONE = 3
};

typedef struct sparse_attn_config {
    int32_t heads;         /* >= 1 */
    int32_t head_dim;      /* 64 or 128 */
    int32_t grid[3];       /* T, H, W: latent token grid, each >= 1 */
    int32_t tile[3];       /* tt, th, tw: tile shape, each >= 1, product B <= 128 */
    int32_t dtype;         /* SPARSE_ATTN_F32 or SPARSE_ATTN_BF16 */
    float softmax_scale;   /* score scale s; 0 selects 1 / sqrt(head_dim) */
    int32_t order;         /* SPARSE_ATTN_ORDER_TILES (0) or SPARSE_ATTN_ORDER_HILBERT */
    int32_t pairing;       /* SPARSE_ATTN_PAIRING_* (0 = AUTO) */
    /* Nonzero runs on the vector-ALU kernel instead of the matrix-core
     * kernels (for comparison and testing), bf16 and fp32 alike. */
    int32_t vector_alu;
} sparse_attn_config;

/*
 * One temporal-distance group of a dual-window mask (Compact Attention
 * page, Fig. 1 caption part (3); Fig. 4 caption).  Tiles are located by
 * (a, b, e) = tile coordinates along (t, y, x).  A query tile i keeps key
 * tile j when |a_i - a_j| lies in [dt_lo, dt_hi] (dt_hi = -1: no upper
 * bound) and, for some w in {0, 1} with ry[w] >= 0 and rx[w] >= 0,
 * |b_i - b_j| <= ry[w] and |e_i - e_j| <= rx[w].  Windows are centred on the
 * query tile and clip at the grid edge; a half-extent of -1 disables the
 * window.  The groups of one head must be sorted, disjoint and satisfy
 * 0 <= dt_lo <= dt_hi (or dt_hi = -1 for the last group only).
 */
typedef struct sparse_attn_window_group {
    int32_t dt_lo, dt_hi;
    int32_t ry[2];
    int32_t rx[2];
} sparse_attn_window_group;

typedef struct sparse_attn_mask {
    int32_t kind; /* SPARSE_ATTN_MASK_BITMAP or SPARSE_ATTN_MASK_DUAL_WINDOW */
    /* BITMAP: device uint8 [heads][nT][nT], row-major (h, i, j); nonzero keeps
     * key tile j for query tile i.  Read during set_mask only. */
    const uint8_t *bitmap;
    /* DUAL_WINDOW: host arrays, copied during set_mask.  groups holds the
     * groups of head 0, then head 1, ...; groups_per_head[h] in 1..MAX_GROUPS. */
    const sparse_attn_window_group *groups;
    const int32_t *groups_per_head;
    /* Upper bound on kept tile pairs over all heads, sizing the index list;
     * <= 0 means heads * nT * nT. */
    int64_t max_nnz;
} sparse_attn_mask;

typedef struct sparse_attn_layout_info {
    int64_t tokens;        /* N = T * H * W */
    int64_t tiles;         /* nT = nt * ny * nx */
    int32_t tile_grid[3];  /* nt, ny, nx = ceil(T / tt), ceil(H / th), ceil(W / tw) */
    int32_t tile_volume;   /* B = tt * th * tw: tokens in a whole tile */
    int64_t slots;         /* N_pad = nT * S: rows of a tile-major tensor */
    int32_t kernel;        /* SPARSE_ATTN_KERNEL_* that forward runs */
    int32_t v_layout;      /* SPARSE_ATTN_LAYOUT_* of the permuted V in the workspace */
    /* Byte offsets of the permuted Q, K, V and of the tile-major output O
     * inside the forward workspace, and the workspace size. */
    size_t ws_offset_q, ws_offset_k, ws_offset_v, ws_offset_o, ws_bytes;
    /* Query-tile pairs of the matrix-core kernel: tiles (2c, 2c + 1) along
     * tile-grid axis pair_axis (0 = t, 1 = y, 2 = x; -1: none) form pair
     * c, numbered raster over pair_grid (the tile grid with that axis halved,
     * rounded up); pairs is pairs per head. */
    int32_t pair_axis;
    int32_t pair_grid[3];
    int64_t pairs;
    int32_t order;         /* SPARSE_ATTN_ORDER_* of the handle */
    /* The pairing in effect (OVERLAP, ALL or NONE; AUTO resolved), or -1
     * for the fp32 matrix-core and vector-ALU kernels. */
    int32_t pairing;
    /* S: slots per tile in the tile-major layout, 128 for the bf16
     * matrix-core kernels, B for the fp32 matrix-core and vector-ALU
     * kernels.  Tile tau owns slots [tau S, tau S + S); empty ones are zero
     * in permuted inputs. */
    int32_t slot_stride;
} sparse_attn_layout_info;

typedef struct sparse_attn_handle sparse_attn_handle;

/*
 * Validate a configuration and plan the tile layout (host only, no device
 * call).  Tiles are numbered raster over the tile grid (t, then y, then x);
 * tiles at the far edges of a grid the tile does not divide are clipped.
 * Each tile owns S consecutive slots (S = 128 on the bf16 matrix-core
 * kernels, B = tt th tw on the fp32 matrix-core and vector-ALU kernels): its
 * c real tokens fill the first c in raster order over the clipped tile, the
 * rest are empty.
 * Errors: INVALID_ARG (null, non-positive sizes, bad dtype, order or pairing),
 * UNSUPPORTED (head_dim not 64/128, B > 128, heads * nT * nT >= 2^31,
 * N >= 2^31, a Hilbert grid side above 2^21).
 * On success *out owns host memory only; release it with sparse_attn_destroy.
 */
int sparse_attn_create(const sparse_attn_config *cfg, sparse_attn_handle **out);

/* Release a handle (host memory only).  NULL is a no-op. */
void sparse_attn_destroy(sparse_attn_handle *h);

/* Describe the planned layout and workspace.  Errors: INVALID_ARG. */
int sparse_attn_layout(const sparse_attn_handle *h, sparse_attn_layout_info *info);

/* Device bytes the compiled-mask buffer needs for at most max_nnz kept tile
 * pairs (<= 0: heads * nT * nT).  With the bf16 matrix-core kernels the buffer
 * holds two index lists of max_nnz entries (rows and query-tile pairs, see
 * sparse_attn_set_mask), otherwise one.  Errors: INVALID_ARG. */
int sparse_attn_mask_bytes(const sparse_attn_handle *h, int64_t max_nnz, size_t *bytes);

/* Device bytes of the forward workspace (permuted Q, K, V and O).
 * Errors: INVALID_ARG. */
int sparse_attn_workspace_bytes(const sparse_attn_handle *h, size_t *bytes);

/* Device bytes of the token-order buffer: 4 N in the Hilbert order (the
 * raster token of each rank, int32), 0 in the tile order.
 * Errors: INVALID_ARG. */
int sparse_attn_order_bytes(const sparse_attn_handle *h, size_t *bytes);

/*
 * Hilbert order: upload the rank -> token map into order_buf (device,
 * caller-owned, 16-byte aligned, at least sparse_attn_order_bytes bytes),
 * which must stay alive and unmodified while the handle moves tokens.
 * Every call that takes a tensor in raster order (forward, the permute and
 * attend stages, the permute hooks) fails with NO_ORDER until this is done.
 * In the tile order it does nothing and succeeds.
 * Errors: INVALID_ARG, WORKSPACE_TOO_SMALL, HIP_ERROR.
 */
int sparse_attn_set_order(sparse_attn_handle *h, void *order_buf, size_t bytes, void *stream);

/*
 * Compile a mask on the GPU into mask_buf: per query-tile row r = h nT + i
 * the kept key tiles in ascending order (row offsets by exclusive sum of row
 * lengths), and a work order of rows by decreasing length, ties by row id.
 * With the bf16 matrix-core kernels it also compiles the same lists for
 * pairs of neighbouring query tiles (union of the two rows, each entry
 * marked with the tiles that keep it), which is what the pair kernel walks.
 * mask_buf (device, caller-owned, at least sparse_attn_mask_bytes(max_nnz)
 * bytes) must stay alive and unmodified while forwards use the mask; calling
 * again replaces the mask.  If the mask keeps more pairs than max_nnz, the
 * index list is truncated (never overrun), forward uses the truncated lists,
 * and sparse_attn_mask_info reports the overflow.
 * Errors: INVALID_ARG (null pointers), BAD_MASK (kind, group count, order or
 * extents), WORKSPACE_TOO_SMALL (bytes), HIP_ERROR.
 */
int sparse_attn_set_mask(sparse_attn_handle *h, const sparse_attn_mask *m, void *mask_buf,
                         size_t bytes, void *stream);

/*
 * Block-sparse attention forward.  q, k, v, o: device [heads][T*H*W][head_dim]
 * in raster token order, element type cfg.dtype; o must not overlap q, k, v
 * or ws, and none of them may overlap ws.  ws: device workspace of at least
 * sparse_attn_workspace_bytes.  Enqueues the permute of K and V to the
 * tile-major layout, then attention over the kept tile pairs, which reads
 * each query row of q and writes its row of o directly (the permute of Q and
 * the unpermute of O are fused into the attention kernels).  Only the K and
 * V regions of ws are used.  The result is bit-identical to the three-stage
 * path below.
 * Errors: INVALID_ARG, NO_MASK, WORKSPACE_TOO_SMALL, HIP_ERROR.
 */
int sparse_attn_forward(sparse_attn_handle *h, const void *q, const void *k, const void *v, void *o,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * sparse_attn_forward that also returns, per query, the log-sum-exp of its
 * kept scores: lse[h][n] = ln sum over kept keys m of exp(s q_n . k_m)
 * (natural log; -infinity for a query whose tile keeps nothing, whose o row
 * is 0).  This is the per-row softmax statistic that the AdaSpa page
 * (abstract) caches across denoising steps: with it, the weight of any key
 * is exp(s q_n . k_m - lse) without another pass.  lse: device fp32
 * [heads][T*H*W] in raster order, 16-byte aligned, overlapping none of q,
 * k, v, o, ws; NULL = none (then this is sparse_attn_forward).  It is
 * computed from the same running max and row sum that normalize o.
 * Errors: as sparse_attn_forward.
 */
int sparse_attn_forward_lse(sparse_attn_handle *h, const void *q, const void *k, const void *v,
                            void *o, float *lse, void *ws, size_t ws_bytes, void *stream);

/*
 * sparse_attn_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation calls).  The permuted K and V go to a
 * library-owned device array of fixed size (SPARSE_ATTN_NOALLOC_SCRATCH_BYTES,
 * 128 MiB; each device that runs the library holds its own copy until the
 * process ends) instead of ws; the call allocates nothing and calls no
 * allocating routine.  The array's device address is looked up on the first
 * call on each device (the device current at the call); the stream must
 * belong to that device.  Same arguments, results and errors as
 * sparse_attn_forward, plus UNSUPPORTED when the permuted K and V need more
 * than the array holds (2 * heads * slots * head_dim * element bytes,
 * each half rounded up to 256 bytes); the scratch check comes before the
 * mask check.  Every call on a device shares that device's array: calls
 * that overlap in time on one device (other streams, other threads) race
 * and must be ordered by the caller.  The array keeps the last call's
 * contents; nothing in it needs to start at zero.
 */
#define SPARSE_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int sparse_attn_forward_noalloc(sparse_attn_handle *h, const void *q, const void *k, const void *v, void *o,
                                void *stream);

/* The two stages of sparse_attn_forward(_lse), callable one by one (same
 * arguments and errors): permute K and V into ws, then attention reading q
 * and writing o (and lse, may be NULL) in raster order. */
int sparse_attn_permute_kv(sparse_attn_handle *h, const void *k, const void *v, void *ws,
                           size_t ws_bytes, void *stream);
int sparse_attn_attend_raster(sparse_attn_handle *h, const void *q, void *o, float *lse, void *ws,
                              size_t ws_bytes, void *stream);

/* The three-stage path, for callers that want the tile-major tensors (the
 * tile selection reads the permuted Q and K): permute Q, K, V into ws;
 * attention from and to ws; unpermute O out of ws.  In order, they give
 * the same o as sparse_attn_forward, bit for bit. */
int sparse_attn_permute_inputs(sparse_attn_handle *h, const void *q, const void *k, const void *v,
                               void *ws, size_t ws_bytes, void *stream);
int sparse_attn_attend(sparse_attn_handle *h, void *ws, size_t ws_bytes, void *stream);
int sparse_attn_unpermute_output(sparse_attn_handle *h, void *ws, size_t ws_bytes, void *o,
                                 void *stream);

/*
 * Tile selection on the GPU: a top-k tile bitmap from Q and K, for
 * sparse_attn_set_mask (SCOPE review page: the abstract names masks built
 * from block-level proxy scores, "The reading" a per-head Top-k count;
 * AdaSpa page, abstract: a blockified pattern).  Score of tile pair (i, j)
 * in head h: softmax scale * qbar_i . kbar_j, with qbar, kbar the fp32 means
 * of the tiles' real tokens; row i keeps the k_per_head[h] key tiles with
 * the largest score, ties to the lower j.
 * Reads the permuted Q and K in ws (call sparse_attn_permute_inputs on ws
 * first) and uses the output region of ws as scratch.  k_per_head: host
 * int32 [heads], each in 0..nT.  bitmap: device uint8 [heads][nT][nT], out.
 * Errors: INVALID_ARG (null pointers, k out of range), UNSUPPORTED (more
 * than 8192 tiles, or tiles too small for the scratch: S * elem < 8 bytes),
 * WORKSPACE_TOO_SMALL, HIP_ERROR.
 */
int sparse_attn_select_topk(sparse_attn_handle *h, const int32_t *k_per_head, void *ws,
                            size_t ws_bytes, uint8_t *bitmap, void *stream);

/*
 * Tile selection with the online per-head Top-k estimate (SCOPE review
 * page, "What carries the argument" and the summary: a hybrid Top-p /
 * fixed Top-k count per query cluster, the head's query-size-weighted
 * average k_head = ceil(sum_c n_c b_c / sum_c n_c), and r_c =
 * max(b_c, k_head); the page's fixed Top-k ratio is 0.1 and its Top-p
 * threshold is not reported).  A query cluster is a query tile here, n_c
 * its real tokens, and the proxy logits are the tile scores of
 * sparse_attn_select_topk.  Per query tile i of head h:
 *   p_i    = the smallest m such that the m largest softmax probabilities
 *            of row i's scores (softmax over all key tiles) sum to at least
 *            rho; 0 when rho <= 0, nT when rho >= 1;
 *   base_i = min(nT, max(p_i, k_fixed));
 *   keep_i = max(base_i, k_head), k_head = ceil(sum_i c_i base_i / N);
 * and row i keeps its keep_i highest-scoring key tiles, ties to the lower
 * j.  rho is applied in fp32 (row sums of fp32 exponentials), the counts
 * are exact integers.  k_fixed: the fixed Top-k floor in key tiles (the
 * page's ratio 0.1 is k_fixed = ceil(0.1 nT)).  Reads the permuted Q and K
 * in ws (call sparse_attn_permute_inputs first) and uses the output region
 * of ws as scratch.  bitmap: device uint8 [heads][nT][nT], out.  base,
 * keep: device int32 [heads][nT], out, or NULL.  None of bitmap, base, keep
 * may overlap ws or each other.
 * Errors: INVALID_ARG (null bitmap, rho not finite, k_fixed outside 0..nT,
 * overlapping buffers), UNSUPPORTED (more than 8192 tiles, or tiles too
 * small for the scratch), WORKSPACE_TOO_SMALL, HIP_ERROR.
 */
int sparse_attn_select_scope(sparse_attn_handle *h, float rho, int32_t k_fixed, void *ws, size_t ws_bytes,
                             uint8_t *bitmap, int32_t *base, int32_t *keep, void *stream);

/*
 * Reference attention mass per tile pair, the input of the offline window
 * search (Compact Attention page, Fig. 1 caption: reference attention mass
 * of query-key regions; Fig. 4 caption: the search keeps the regions that
 * hold most of each head's attention mass).  With p(n, .) the softmax of
 * s q_n . k over ALL N keys,
 *     mass[h][i][j] = (1 / c_i) sum_{n in tile i} sum_{m in tile j} p(n, m),
 * the mean over the real queries of tile i of the mass they give tile j
 * (each row sums to 1).  q, k: raster [heads][N][head_dim] bf16; ws: the
 * forward workspace (its Q and K regions are overwritten); mass: device fp32
 * [heads][nT][nT], out.  This is dense work (two passes of Q K^T over every
 * key); it is meant for offline calibration, not the forward path.
 * Errors: INVALID_ARG, UNSUPPORTED (needs the matrix-core path: bf16 and
 * not vector_alu), WORKSPACE_TOO_SMALL, NO_ORDER, HIP_ERROR.
 */
int sparse_attn_tile_mass(sparse_attn_handle *h, const void *q, const void *k, void *ws,
                          size_t ws_bytes, float *mass, void *stream);

/*
 * Offline dual-window search on the host (Compact Attention page, Fig. 3
 * caption: windows shrunk under a recall constraint tau and a cost
 * constraint lambda; Fig. 4 caption: starting from full coverage in every
 * temporal-distance group; Fig. 1 caption part (3): two windows per group).
 * The pages give no formula; this is the reading implemented:
 *   - Tile pair (i, j) weighs w = round(mass[i][j] c_i 2^24) and costs
 *     c_i c_j.  A head's recall is its kept weight over all its weight, its
 *     cost the kept cost over N^2.
 *   - The groups' [dt_lo, dt_hi] come from groups_in (windows ignored).  A
 *     group's kept offsets (|db|, |de|) are the union of a wide rectangle
 *     (ry y, rx X) and a tall one (ry Y, rx x), -1 <= y <= Y <= ny - 1 and
 *     -1 <= x <= X <= nx - 1: window 0 = (y, X), window 1 = (Y, x).
 *   - Start: every group full (y = Y = ny - 1, x = X = nx - 1).  Moves of a
 *     group, numbered: 0 notch a rectangle's corner (y = Y and x = X:
 *     y -= 1, x -= 1); 1 y -= 1; 2 x -= 1; 3 Y -= 1 (y = min(y, Y));
 *     4 X -= 1 (x = min(x, X)).  A move that uncovers no offset is not a
 *     candidate.  A candidate is admissible when the kept weight stays at
 *     least ceil(tau * total weight) and lost weight / total weight is at
 *     most lambda * saved cost / N^2 (lambda = INFINITY: no such limit).
 *   - Each step applies the admissible candidate of any group with the
 *     least lost weight per saved cost (a move that saves no cost comes
 *     first), ties to the larger saved cost, the lower group, the lower
 *     move; the search stops when none is admissible.
 * mass: host fp32 [heads][nT][nT] (sparse_attn_tile_mass copied back);
 * groups_in / groups_per_head: as for a dual-window mask; groups_out: host,
 * same count, the searched windows; recall, cost: host [heads].  Host only,
 * synchronous.  Errors: INVALID_ARG (null, tau outside [0, 1], lambda <=
 * 0), BAD_MASK (groups).
 */
int sparse_attn_search_windows(sparse_attn_handle *h, const float *mass,
                               const sparse_attn_window_group *groups_in, const int32_t *groups_per_head,
                               double tau, double lambda, sparse_attn_window_group *groups_out,
                               double *recall, double *cost);

/*
 * Test hooks.
 * sparse_attn_permute: src [heads][N][head_dim] raster -> dst in `layout`
 *   (SPARSE_ATTN_LAYOUT_*), empty slots zero.  dst holds heads * nT * S *
 *   head_dim elements (S = the layout's slot_stride).
 * sparse_attn_unpermute: src [heads][nT * S][head_dim] rows -> dst
 *   [heads][N][head_dim] raster; empty slots are not read.
 * sparse_attn_read_index_lists: copy the compiled row offsets (int32
 *   [heads nT + 1]), index list (int32, first min(nnz, cols_capacity)
 *   entries) and work order (int32 [heads nT]) into device buffers.
 * sparse_attn_read_pair_lists: the same for the query-tile pair lists of
 *   the bf16 matrix-core kernels (rows r = h * pairs + p), plus flag (int32
 *   [heads * pairs]: 1 when the pair kernel serves the pair, whose list is
 *   then the union of its two tiles' rows; 0 when the row kernel serves its
 *   tiles and its list is empty).  Each entry packs key tile j (bits 0-15),
 *   its real token count (bits 16-23) and whether the pair's first and
 *   second tile keep it (bits 24, 25).  UNSUPPORTED for the fp32
 *   matrix-core and vector-ALU kernels.
 * sparse_attn_mask_info: synchronizes `stream`, then reports the number of
 *   kept pairs and whether the index list overflowed its capacity.
 * Errors: INVALID_ARG, NO_MASK (index lists), UNSUPPORTED, HIP_ERROR.
 */
int sparse_attn_permute(sparse_attn_handle *h, const void *src, void *dst, int32_t layout,
                        void *stream);
int sparse_attn_unpermute(sparse_attn_handle *h, const void *src, void *dst, void *stream);
int sparse_attn_read_index_lists(sparse_attn_handle *h, int32_t *row_ptr, int32_t *cols,
                                 int64_t cols_capacity, int32_t *order, void *stream);
int sparse_attn_read_pair_lists(sparse_attn_handle *h, int32_t *row_ptr, int32_t *cols,
                                int64_t cols_capacity, int32_t *order, int32_t *flag, void *stream);
int sparse_attn_mask_info(sparse_attn_handle *h, int64_t *nnz, int32_t *overflow, void *stream);

/*
 * Diagnostic, not part of the attention path: how fast this GPU runs the
 * instruction mix of one attention stage with nothing else in the way, as
 * context for the attention kernels' fraction of the published matrix peak
 * (the chip's clock, and so its rate, follows the power that work draws).
 * Each wave runs `iters` stages of an attention wave's work on a 64-key
 * stage held in LDS: 16 v_mfma_f32_32x32x16_bf16 products of S^T = K Q^T,
 * the kernels' online-softmax step on the 32 x 64 scores, 16 products of
 * O^T += V^T P^T, and workgroup barriers; head_dim 128, operands
 * pseudo-random bf16 in [-1, 1), no global memory traffic inside the loop.
 * One stage of one wave is 32 products of 32 x 32 x 16, 2^20 FLOP.
 *   pingpong 0: cus * waves_per_simd workgroups of 4 waves (one per SIMD),
 *     waves_per_simd of them resident per compute unit when cus is the
 *     GPU's compute-unit count; the waves of a SIMD run unsynchronised, one
 *     barrier per stage (the row kernel's schedule at waves_per_simd 2);
 *   pingpong 1 (waves_per_simd must be 2): cus workgroups of 8 waves, two
 *     per SIMD, waves 4-7 half a step behind waves 0-3 through one extra
 *     barrier, two barriers per stage (the pair kernel's schedule).
 *   waves_per_simd: 1, 2 or 3; cus: 1..65536; iters: 1..2^20 (a launch of
 *     2^20 stages runs for a few seconds);
 *   cycles: device int64 [cus * waves_per_simd * 4], out: each wave's
 *     shader-clock cycles over its loop (s_memtime);
 *   sink: device fp32 [cus * waves_per_simd * 256], out: a per-lane sum of
 *     the results (keeps the work live; its value means nothing).
 * Asynchronous on `stream`.  Errors: INVALID_ARG, HIP_ERROR (message in
 * sparse_attn_last_error(NULL)).
 */
int sparse_attn_mix_probe(int32_t waves_per_simd, int32_t pingpong, int32_t cus, int32_t iters, int64_t *cycles,
                          float *sink, void *stream);

/* Static description of a status code. */
const char *sparse_attn_status_string(int status);

/* Message of the last failed call on this handle ("" if none).  The string
 * stays valid until the next call on the handle.  NULL handle: the message of
 * the last failed sparse_attn_create on this thread. */
const char *sparse_attn_last_error(const sparse_attn_handle *h);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
