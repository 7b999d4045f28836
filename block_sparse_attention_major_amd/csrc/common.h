// Internal definitions shared by the HIP kernels and the host library.
//
// Tile layout (Compact Attention page, abstract: one tile-aligned mask
// family; Fig. 3 caption: masks run in block-sparse attention kernels).  The
// T x H x W token grid (raster token id n = (t H + y) W + x) is cut into
// tt x th x tw tiles, numbered raster over the tile grid (nt, ny, nx).  Tiles
// at the far edges are clipped.  Tile tau owns slots [tau S, tau S + S) of
// the tile-major layout: S = 128 for the bf16 matrix-core kernels (whatever
// the tile volume tt th tw <= 128), S = tt th tw for the vector-ALU kernel.
// Its c_tau real tokens fill the first c_tau slots in raster order over the
// clipped tile, and the remaining slots are empty (zero in permuted inputs,
// never read back from outputs).  One tile is one block of the attention
// kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa {

struct Layout {
    int T, H, W;      // token grid
    int tt, th, tw;   // tile shape
    int nt, ny, nx;   // tile grid
    int nT;           // tiles
    int S;            // slots per tile
    int heads;
    int D;            // head dim
    long long N;      // tokens
    long long Npad;   // slots = nT * S
    // Query-tile pairs.  The matrix-core kernel runs two query tiles of one
    // head per workgroup, over the union of their key lists.  Tiles pair up
    // along axis pax (0 = t, 1 = y, 2 = x) as coordinates (2c, 2c + 1); a
    // last tile on an odd axis is alone.  pax = -1: no pairing.
    int pax;
    int pn[3];        // pair grid (tile grid with the paired axis halved)
    int nP;           // pairs per head
    // Hilbert order: the token grid above is the 1 x 1 x N sequence of
    // tokens in Hilbert rank order, cut into tiles of 1 x 1 x B, and
    // seq_tok[p] (device, [N]) is the raster token at sequence position p.
    // Null for the tile-box order, where positions are raster tokens.
    const int *seq_tok;
};

// Clipped extents of tile tau along t, y, x.
struct TileBox {
    int a, b, e;      // tile coordinates
    int et, ey, ex;   // clipped extents
};

__host__ __device__ inline TileBox tile_box(const Layout &L, int tau)
{
    TileBox r;
    r.a = tau / (L.ny * L.nx);
    r.b = (tau / L.nx) % L.ny;
    r.e = tau % L.nx;
    r.et = min(L.tt, L.T - r.a * L.tt);
    r.ey = min(L.th, L.H - r.b * L.th);
    r.ex = min(L.tw, L.W - r.e * L.tw);
    return r;
}

__host__ __device__ inline int tile_real_count(const Layout &L, int tau)
{
    TileBox r = tile_box(L, tau);
    return r.et * r.ey * r.ex;
}

// Grid position of real slot s (0 <= s < c_tau) of the tile with box bx:
// the raster token in the tile-box order, the sequence position in the
// Hilbert order.
__host__ __device__ inline int slot_token(const Layout &L, const TileBox &bx, int s)
{
    const int plane = bx.ey * bx.ex;
    const int lt = s / plane, rem = s - lt * plane;
    const int ly = rem / bx.ex, lx = rem - ly * bx.ex;
    return ((bx.a * L.tt + lt) * L.H + bx.b * L.th + ly) * L.W + bx.e * L.tw + lx;
}

// Raster token of grid position p (see Layout::seq_tok).
__device__ inline int position_token(const Layout &L, int p) { return L.seq_tok ? L.seq_tok[p] : p; }

// Raster token of real slot s of tile tau.
__device__ inline int raster_token(const Layout &L, int tau, int s)
{
    return position_token(L, slot_token(L, tile_box(L, tau), s));
}

// The query tiles of pair pr (raster over the pair grid); t2 = -1 when the
// first tile is alone.
struct TilePair {
    int t1, t2;
};

// The pair holding query tile i (inverse of pair_tiles).
__host__ __device__ inline int tile_pair(const Layout &L, int i)
{
    int a = i / (L.ny * L.nx);
    int b = (i / L.nx) % L.ny;
    int e = i % L.nx;
    if (L.pax == 0)
        a >>= 1;
    else if (L.pax == 1)
        b >>= 1;
    else if (L.pax == 2)
        e >>= 1;
    return (a * L.pn[1] + b) * L.pn[2] + e;
}

__host__ __device__ inline TilePair pair_tiles(const Layout &L, int pr)
{
    int a = pr / (L.pn[1] * L.pn[2]);
    int b = (pr / L.pn[2]) % L.pn[1];
    int e = pr % L.pn[2];
    int a2 = a, b2 = b, e2 = e;
    bool two = false;
    if (L.pax == 0) {
        a *= 2;
        a2 = a + 1;
        two = a2 < L.nt;
    } else if (L.pax == 1) {
        b *= 2;
        b2 = b + 1;
        two = b2 < L.ny;
    } else if (L.pax == 2) {
        e *= 2;
        e2 = e + 1;
        two = e2 < L.nx;
    }
    TilePair r;
    r.t1 = (a * L.ny + b) * L.nx + e;
    r.t2 = two ? (a2 * L.ny + b2) * L.nx + e2 : -1;
    return r;
}

// A pair-list entry packs the key tile j (bits 0-15; the host keeps
// nT <= 46340), its real token count c_j (bits 16-23, at most 128) and
// whether the first and the second query tile of the pair keep it (bits 24
// and 25).
constexpr int kPairCountShift = 16;
constexpr int kPairBitsShift = 24;
__host__ __device__ inline int pair_entry(int j, int c, int bits)
{
    return j | (c << kPairCountShift) | (bits << kPairBitsShift);
}

// Division of 0 <= n < 2^31 by a fixed divisor 1 <= d < 2^31 with one
// multiply-high, add and shift: the round-up method of Granlund and
// Montgomery, "Division by invariant integers using multiplication" (1994):
// s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1, q = (mulhi(n, m) + n) >> s.
struct FastDiv {
    uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t s = 0;
    while ((1ull << s) < d)
        ++s;
    const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, s};
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv &f)
{
    return (__umulhi(n, f.m) + n) >> f.s;
}

constexpr float kLn2 = 0.69314718055994531f;

// Round a byte count up to a 256-byte boundary.
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// Kernel launchers (each returns the launch status).

// Raster rows [heads][N][D] -> tile-major rows [heads][Npad][D], empty slots 0.
hipError_t launch_permute_rows(const Layout &L, int elem_bytes, const void *src, void *dst,
                               hipStream_t s);
// Raster rows -> per-tile transposed [heads][nT][D][B] (bf16 only).
hipError_t launch_permute_tile_columns(const Layout &L, const void *src, void *dst, hipStream_t s);
// Tile-major rows [heads][Npad][D] -> raster rows [heads][N][D].
hipError_t launch_unpermute_rows(const Layout &L, int elem_bytes, const void *src, void *dst,
                                 hipStream_t s);

// Compiled mask buffers inside the caller's mask buffer.
struct MaskBuffers {
    int *row_ptr;   // [R + 1]
    int *len;       // [R]
    int *order;     // [R]
    int *chunk;     // [nchunks][nT + 1]: per-chunk length histogram, then bases
    int *bucket;    // [nT + 1]
    int *status;    // [0] = nnz, [1] = overflow flag
    int *groups;    // [heads * MAX_GROUPS][6]
    int *group_off; // [heads + 1]
    int *cols;      // [cap]
    long long cap;
    int R;
    int nchunks;
    int pair;       // 0: rows r = h nT + i; 1: pairs r = h nP + pr (entries carry keep bits)
    int *flag;      // pairs only, [R]: 1 = the pair kernel serves the pair (see kPairNum)
    int pairing;    // pairs only: SPARSE_ATTN_PAIRING_OVERLAP, _ALL or _NONE (AUTO resolved)
    FastDiv dplane; // ny * nx: tiles per tile-grid plane
    FastDiv drow;   // nx: tiles per tile-grid row
};

// A pair of query tiles goes to the pair kernel when the union of their key
// lists is at most kPairNum / kPairDen of the two lists' total length (every
// kept key tile of the union is then loaded once for both tiles often enough
// to pay for the steps where only one tile computes); otherwise both tiles
// go to the row kernel.  A pair with no kept tiles is served by the pair
// kernel (it writes zeros).
constexpr int kPairNum = 7, kPairDen = 10;

// SPARSE_ATTN_PAIRING_AUTO: a layout with at most kSmallLayoutPairs
// query-tile pairs over all heads (a few per compute unit) sends every tile
// to the row kernel.  With so little work the GPU is not filled, and the
// row kernel's one-tile workgroups, two per compute unit, balance it better
// than pairs of tiles: more, shorter work items, and no union of two lists.
constexpr long long kSmallLayoutPairs = 1024;

constexpr int kMaskChunk = 256;  // rows per chunk of the order sort

// Compiles the mask into mb; then, when pb.R > 0, into the pair lists pb
// (which share mb's groups).
hipError_t launch_compile_mask(const Layout &L, int kind, const uint8_t *bitmap,
                               const MaskBuffers &mb, const MaskBuffers &pb, hipStream_t s);

// One compiled set of index lists.
struct ListSet {
    const int *row_ptr;
    const int *cols;
    const int *order;
    long long cap;      // valid entries of cols
};

struct AttnParams {
    const void *q;      // tile-major rows, or raster rows when raster = 1
    const void *k;      // tile-major rows
    const void *v;      // tile-major rows (generic) or tile columns (MFMA)
    void *o;            // tile-major rows, or raster rows when raster = 1
    int raster;         // 1: q is read from and o written to [heads][N][D] in raster
                        //    order (real slots only); 0: both tile-major
    float *lse;         // null, or [heads][N] raster: ln sum over kept keys of exp(score)
    ListSet rows;       // per query tile
    ListSet pairs;      // per query-tile pair (matrix-core kernels only)
    const int *pair_flag;  // [heads nP] (matrix-core kernels only)
    float scale_log2;   // softmax scale * log2(e)
    int xcd_chunk;      // rows per XCD chunk of the work order (0: plain order)
    FastDiv div_plane;  // ny * nx: tiles per tile-grid plane
    FastDiv div_row;    // nx: tiles per tile-grid row
};

// bf16 matrix-core kernels, 128 slots per tile (tile volume <= 128), D in
// {64, 128}: the pair kernel over accepted query-tile pairs, then the row
// kernel over the other query tiles.
hipError_t launch_attention_mfma(const Layout &L, const AttnParams &p, hipStream_t s);
hipError_t launch_attention_rows(const Layout &L, const AttnParams &p, hipStream_t s);
// fp32 matrix-core kernel (one query tile per workgroup over the row lists),
// D in {64, 128}; needs N_pad D 4 bytes per head below 2^31.
hipError_t launch_attention_f32(const Layout &L, const AttnParams &p, hipStream_t s);
// Tile selection from the tile-major Q and K: fp32 tile means into qbar,
// kbar ([heads][nT][D]), then per row the kh[h] best-scoring key tiles
// (ties to the lower tile) into bitmap [heads][nT][nT].  nT <= kSelectMaxTiles.
constexpr int kSelectMaxTiles = 8192;
hipError_t launch_select_topk(const Layout &L, int elem_bytes, const void *q, const void *k,
                              const int *kh, float scale, float *qbar, float *kbar, uint8_t *bitmap,
                              hipStream_t s);
// The same with the per-head Top-k estimate: per row the hybrid Top-p /
// fixed Top-k base count into base [heads][nT] (rho: Top-p threshold,
// k_fixed: the fixed count), the per-head estimate and final counts
// max(base, k_head) into keep [heads][nT], then per row its keep best key
// tiles into bitmap.
hipError_t launch_select_scope(const Layout &L, int elem_bytes, const void *q, const void *k, float scale,
                               float rho, int k_fixed, float *qbar, float *kbar, int *base, int *keep,
                               uint8_t *bitmap, hipStream_t s);

// Full-attention mass per tile pair from the tile-major bf16 Q and K (B ==
// 128): mass [heads][nT][nT], row (h, i) = mean over tile i's real queries
// of the softmax mass on each key tile.
hipError_t launch_tile_mass(const Layout &L, const void *q, const void *k, float scale_log2, float *mass,
                            hipStream_t s);

// fp32 vector-ALU kernel for any supported shape; elem_bytes 4 (fp32) or 2 (bf16).
hipError_t launch_attention_generic(const Layout &L, int elem_bytes, const AttnParams &p,
                                    hipStream_t s);

// Greedy dual-window search of one head on the host (mass A [nT][nT] fp32;
// G validated groups; writes G groups with their windows, recall and cost).
int search_head(const Layout &L, const float *A, const sparse_attn_window_group *gin, int G, double tau,
                double lambda, sparse_attn_window_group *gout, double *recall, double *cost);

}  // namespace sa
