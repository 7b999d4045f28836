// Mask compiler: tile bitmap or dual-window spec -> per-query-tile index
// lists of kept key tiles, and a longest-first work order.
//
// The pages' pipeline precomputes a mask per head and loads it into the
// block-sparse attention kernel, reusing it over several denoising steps
// (Compact Attention page, Fig. 3 caption), so this runs once per mask.
// Dual windows follow the reading given at sparse_attn_window_group: keep
// (i -> j) when the tile-t distance lies in a group and the (y, x) offset
// lies inside one of that group's two centred windows (Fig. 1 caption part
// (3), Fig. 4 caption).
//
// Every output is deterministic: row lengths and histograms are counts, the
// index list is written by an ordered ballot compaction, and the work order
// is a stable counting sort by decreasing length.
//
// Rows r = h nT + i.  Stages:
//   zero   : clear the per-chunk length histograms and the status words
//   count  : one wave per row -> len[r]; histogram of lengths per 256-row chunk
//   scan   : one workgroup -> row_ptr (exclusive sum of len), nnz, overflow;
//            bucket starts of each length in decreasing order; per-chunk bases
//   fill   : one wave per row -> ascending key-tile ids
//   order  : one workgroup per chunk -> order[base + rank among equal lengths]
//
// The matrix-core path also gets pair lists: the same stages run over
// query-tile pairs r = h nP + pr (pair_tiles), keeping key tile j when
// either tile of the pair keeps it, and each entry carries which of the two
// does (pair_entry: j, its real token count, and the keep bits).  The count
// stage also decides, per pair, whether the pair kernel serves it (flag;
// see kPairNum); a pair it does not serve gets an empty list.  The row
// lists stay the mask's definitive form (they are what the index-list hook
// returns).
#include "common.h"

namespace sa {

namespace {

constexpr int kWave = 64;

struct RowCtx {
    int ai, bi, ei;  // query tile coordinates
};

// The window groups of one head, read once per list into registers:
// rows of (dt_lo, dt_hi, ry0, ry1, rx0, rx1).
struct Windows {
    int n;
    int g[SPARSE_ATTN_MAX_GROUPS][6];
};

// Tile coordinates (a, b, e) of tile j, by multiply-high division.
__device__ __forceinline__ void tile_coords(const Layout &L, const MaskBuffers &mb, int j, int &a, int &b,
                                            int &e)
{
    a = (int)fast_div((uint32_t)j, mb.dplane);
    const int rem = j - a * L.ny * L.nx;
    b = (int)fast_div((uint32_t)rem, mb.drow);
    e = rem - b * L.nx;
}

__device__ __forceinline__ RowCtx tile_ctx(const Layout &L, const MaskBuffers &mb, int i)
{
    RowCtx c;
    tile_coords(L, mb, i, c.ai, c.bi, c.ei);
    return c;
}

__device__ __forceinline__ bool window_keeps(const RowCtx &c, const Windows &w, int aj, int bj, int ej)
{
    const int dt = abs(c.ai - aj), dy = abs(c.bi - bj), dx = abs(c.ei - ej);
#pragma unroll
    for (int g = 0; g < SPARSE_ATTN_MAX_GROUPS; ++g) {
        if (g < w.n) {
            const int *G = w.g[g];
            if (dt < G[0] || (G[1] >= 0 && dt > G[1]))
                continue;
            if (G[2] >= 0 && G[4] >= 0 && dy <= G[2] && dx <= G[4])
                return true;
            if (G[3] >= 0 && G[5] >= 0 && dy <= G[3] && dx <= G[5])
                return true;
        }
    }
    return false;
}

// The query tiles behind list r: one tile for a row list, two (t2 = -1: one)
// for a pair list, and (window masks) the head's groups.
struct ListRow {
    int h, t1, t2;
    RowCtx c1, c2;
    Windows w;
};

template <int KIND>
__device__ __forceinline__ ListRow list_row(const Layout &L, const MaskBuffers &mb, int r)
{
    ListRow q;
    if (mb.pair) {
        q.h = r / L.nP;
        const TilePair tp = pair_tiles(L, r - q.h * L.nP);
        q.t1 = tp.t1;
        q.t2 = tp.t2;
    } else {
        q.h = r / L.nT;
        q.t1 = r - q.h * L.nT;
        q.t2 = -1;
    }
    q.c1 = tile_ctx(L, mb, q.t1);
    q.c2 = tile_ctx(L, mb, q.t2 >= 0 ? q.t2 : q.t1);
    q.w.n = 0;
    if (KIND == 1) {
        const int g0 = mb.group_off[q.h];
        q.w.n = mb.group_off[q.h + 1] - g0;
#pragma unroll
        for (int g = 0; g < SPARSE_ATTN_MAX_GROUPS; ++g)
#pragma unroll
            for (int k = 0; k < 6; ++k)
                q.w.g[g][k] = g < q.w.n ? mb.groups[6 * (g0 + g) + k] : 0;
    }
    return q;
}

// Keep bits of key tile j for list r: bit 0 = first query tile, bit 1 =
// second.  A row list only has bit 0.
template <int KIND>
__device__ __forceinline__ int keep_bits(const Layout &L, const MaskBuffers &mb,
                                         const uint8_t *__restrict__ bitmap, const ListRow &q, int j)
{
    if (KIND == 0) {
        const uint8_t *row = bitmap + (long long)q.h * L.nT * L.nT;
        int bits = row[(long long)q.t1 * L.nT + j] != 0 ? 1 : 0;
        if (q.t2 >= 0 && row[(long long)q.t2 * L.nT + j] != 0)
            bits |= 2;
        return bits;
    }
    int aj, bj, ej;
    tile_coords(L, mb, j, aj, bj, ej);
    int bits = window_keeps(q.c1, q.w, aj, bj, ej) ? 1 : 0;
    if (q.t2 >= 0 && window_keeps(q.c2, q.w, aj, bj, ej))
        bits |= 2;
    return bits;
}

__global__ void zero_kernel(int *__restrict__ p, long long n)
{
    for (long long u = blockIdx.x * (long long)blockDim.x + threadIdx.x; u < n;
         u += (long long)gridDim.x * blockDim.x)
        p[u] = 0;
}

template <int KIND>
__global__ __launch_bounds__(256) void count_kernel(Layout L, MaskBuffers mb,
                                                    const uint8_t *__restrict__ bitmap)
{
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= mb.R)
        return;
    const int lane = threadIdx.x & 63;
    const ListRow q = list_row<KIND>(L, mb, r);
    // n: list length (union for a pair); n12: kept entries of each tile
    // summed (a pair's two row lengths).
    int n = 0, n12 = 0;
    for (int j = lane; j < L.nT; j += kWave) {
        const int kb = keep_bits<KIND>(L, mb, bitmap, q, j);
        n += kb ? 1 : 0;
        n12 += (kb & 1) + (kb >> 1);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        n += __shfl_xor(n, off);
        n12 += __shfl_xor(n12, off);
    }
    if (mb.pair) {
        const int accept = mb.pairing == SPARSE_ATTN_PAIRING_ALL    ? 1
                           : mb.pairing == SPARSE_ATTN_PAIRING_NONE ? 0
                           : (long long)n * kPairDen <= (long long)kPairNum * n12 ? 1 : 0;
        if (lane == 0)
            mb.flag[r] = accept;
        if (!accept)
            n = 0;  // the row kernel serves both tiles
    }
    if (lane == 0) {
        mb.len[r] = n;
        atomicAdd(&mb.chunk[(long long)(r / kMaskChunk) * (L.nT + 1) + n], 1);
    }
}

// Exclusive scan of x[0..n) into y[0..n) (y may alias x) by one workgroup of
// 1024 threads; returns the total to every thread.  `rev` reads and writes
// x[n - 1 - u] for u = 0..n-1 (a scan in decreasing index order).
__device__ long long block_exclusive_scan(const int *x, int *y, long long n, bool rev,
                                          long long *lds)
{
    const int t = threadIdx.x, nt = blockDim.x;
    const long long seg = (n + nt - 1) / nt;
    const long long lo = min(n, t * seg), hi = min(n, lo + seg);
    long long s = 0;
    for (long long u = lo; u < hi; ++u)
        s += x[rev ? n - 1 - u : u];
    lds[t] = s;
    __syncthreads();
    // Hillis-Steele inclusive scan of the per-thread sums.
    for (int off = 1; off < nt; off <<= 1) {
        long long add = t >= off ? lds[t - off] : 0;
        __syncthreads();
        lds[t] += add;
        __syncthreads();
    }
    long long run = lds[t] - s;
    const long long total = lds[nt - 1];
    for (long long u = lo; u < hi; ++u) {
        const long long idx = rev ? n - 1 - u : u;
        const int v = x[idx];
        y[idx] = (int)run;
        run += v;
    }
    __syncthreads();
    return total;
}

__global__ __launch_bounds__(1024) void scan_kernel(Layout L, MaskBuffers mb)
{
    __shared__ long long lds[1024];
    // Row offsets.
    const long long nnz = block_exclusive_scan(mb.len, mb.row_ptr, mb.R, false, lds);
    if (threadIdx.x == 0) {
        mb.row_ptr[mb.R] = (int)nnz;
        mb.status[0] = (int)nnz;
        mb.status[1] = nnz > mb.cap ? 1 : 0;
    }
    // Rows per length, then bucket starts in decreasing length order.
    const int nL = L.nT + 1;
    // (Threads take consecutive lengths, so each chunk row is read
    // coalesced; the loop is unrolled so several reads are in flight.)
    for (int len = threadIdx.x; len < nL; len += blockDim.x) {
        int tot = 0;
#pragma unroll 8
        for (int c = 0; c < mb.nchunks; ++c)
            tot += mb.chunk[(long long)c * nL + len];
        mb.bucket[len] = tot;
    }
    __threadfence_block();
    __syncthreads();
    block_exclusive_scan(mb.bucket, mb.bucket, nL, true, lds);
    __threadfence_block();
    __syncthreads();
    // Base of each (chunk, length): bucket start + rows of that length in
    // earlier chunks.
    constexpr int kBatch = 8;
    for (int len = threadIdx.x; len < nL; len += blockDim.x) {
        int run = mb.bucket[len];
        for (int c0 = 0; c0 < mb.nchunks; c0 += kBatch) {
            int x[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                x[u] = c0 + u < mb.nchunks ? mb.chunk[(long long)(c0 + u) * nL + len] : 0;
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (c0 + u < mb.nchunks)
                    mb.chunk[(long long)(c0 + u) * nL + len] = run;
                run += x[u];
            }
        }
    }
}

template <int KIND>
__global__ __launch_bounds__(256) void fill_kernel(Layout L, MaskBuffers mb,
                                                   const uint8_t *__restrict__ bitmap)
{
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= mb.R)
        return;
    if (mb.pair && !mb.flag[r])
        return;  // no list: the row kernel serves both tiles
    const int lane = threadIdx.x & 63;
    const ListRow q = list_row<KIND>(L, mb, r);
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    long long base = mb.row_ptr[r];
    for (int j0 = 0; j0 < L.nT; j0 += kWave) {
        const int j = j0 + lane;
        const int kb = j < L.nT ? keep_bits<KIND>(L, mb, bitmap, q, j) : 0;
        const unsigned long long bits = __ballot(kb != 0);
        const long long pos = base + __popcll(bits & below);
        if (kb && pos < mb.cap)
            mb.cols[pos] = mb.pair ? pair_entry(j, tile_real_count(L, j), kb) : j;
        base += __popcll(bits);
    }
}

__global__ __launch_bounds__(kMaskChunk) void order_kernel(Layout L, MaskBuffers mb)
{
    __shared__ int lens[kMaskChunk];
    const int t = threadIdx.x;
    const int r = blockIdx.x * kMaskChunk + t;
    const int len = r < mb.R ? mb.len[r] : -1;
    lens[t] = len;
    __syncthreads();
    if (r >= mb.R)
        return;
    int rank = 0;
    for (int u = 0; u < t; ++u)
        rank += lens[u] == len ? 1 : 0;
    const int base = mb.chunk[(long long)blockIdx.x * (L.nT + 1) + len];
    mb.order[base + rank] = r;
}

}  // namespace

namespace {

hipError_t compile_lists(const Layout &L, int kind, const uint8_t *bitmap, const MaskBuffers &mb,
                         hipStream_t s)
{
    const long long nchunk_words = (long long)mb.nchunks * (L.nT + 1);
    hipLaunchKernelGGL(zero_kernel, dim3(256), dim3(256), 0, s, mb.chunk, nchunk_words);
    const dim3 rows_grid((mb.R + 3) / 4);
    if (kind == 0)
        hipLaunchKernelGGL(count_kernel<0>, rows_grid, dim3(256), 0, s, L, mb, bitmap);
    else
        hipLaunchKernelGGL(count_kernel<1>, rows_grid, dim3(256), 0, s, L, mb, bitmap);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, L, mb);
    if (kind == 0)
        hipLaunchKernelGGL(fill_kernel<0>, rows_grid, dim3(256), 0, s, L, mb, bitmap);
    else
        hipLaunchKernelGGL(fill_kernel<1>, rows_grid, dim3(256), 0, s, L, mb, bitmap);
    hipLaunchKernelGGL(order_kernel, dim3(mb.nchunks), dim3(kMaskChunk), 0, s, L, mb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_compile_mask(const Layout &L, int kind, const uint8_t *bitmap,
                               const MaskBuffers &mb, const MaskBuffers &pb, hipStream_t s)
{
    // Status words of both list sets share one 16-word block.
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(64), 0, s, mb.status, 16ll);
    hipError_t e = compile_lists(L, kind, bitmap, mb, s);
    if (e == hipSuccess && pb.R > 0)
        e = compile_lists(L, kind, bitmap, pb, s);
    return e;
}

}  // namespace sa
