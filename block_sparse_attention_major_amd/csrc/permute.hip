// Tile-major token permutation and its inverse.
//
// A tile's real tokens are et * ey runs of ex tokens that are contiguous in
// raster order, and land in contiguous slots.  So one workgroup per
// (head, tile) copies each run as one contiguous block of 16-byte vectors:
// no per-element index arithmetic, fully coalesced reads and writes.  In the
// Hilbert order each slot's row is fetched from its own raster position
// (whole rows, still 16-byte vectors).  Both kernels are bound by HBM
// bandwidth.
#include "common.h"

namespace sa {

namespace {

constexpr int kThreads = 256;

// Copies one run of `nvec` 16-byte vectors.
__device__ __forceinline__ void copy_run(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                         int nvec)
{
    for (int v = threadIdx.x; v < nvec; v += kThreads)
        dst[v] = src[v];
}

// dir = 0: raster -> tile-major (and zero the empty slots); dir = 1: back.
template <int DIR>
__global__ __launch_bounds__(kThreads) void permute_rows_kernel(Layout L, int vpr,
                                                                const uint4 *__restrict__ src,
                                                                uint4 *__restrict__ dst)
{
    const int h = blockIdx.x / L.nT;
    const int tau = blockIdx.x - h * L.nT;
    const TileBox bx = tile_box(L, tau);
    const long long raster0 = (long long)h * L.N;
    const long long slot0 = (long long)h * L.Npad + (long long)tau * L.S;
    if (L.seq_tok) {
        // Hilbert order: consecutive slots hold tokens scattered over the
        // raster, so each slot row is copied on its own (still 16-byte
        // vectors, whole rows per group of threads).
        const int c = bx.et * bx.ey * bx.ex;
        for (int u = threadIdx.x; u < c * vpr; u += kThreads) {
            const int s = u / vpr, w = u - s * vpr;
            const long long n = raster0 + L.seq_tok[slot_token(L, bx, s)];
            if (DIR == 0)
                dst[(slot0 + s) * vpr + w] = src[n * vpr + w];
            else
                dst[n * vpr + w] = src[(slot0 + s) * vpr + w];
        }
    } else {
        for (int lt = 0; lt < bx.et; ++lt) {
            for (int ly = 0; ly < bx.ey; ++ly) {
                const int t = bx.a * L.tt + lt, y = bx.b * L.th + ly, x = bx.e * L.tw;
                const long long n0 = raster0 + ((long long)t * L.H + y) * L.W + x;
                const long long p0 = slot0 + (long long)(lt * bx.ey + ly) * bx.ex;
                if (DIR == 0)
                    copy_run(src + n0 * vpr, dst + p0 * vpr, bx.ex * vpr);
                else
                    copy_run(src + p0 * vpr, dst + n0 * vpr, bx.ex * vpr);
            }
        }
    }
    if (DIR == 0) {
        const int c = bx.et * bx.ey * bx.ex;
        uint4 *pad = dst + (slot0 + c) * vpr;
        const int nvec = (L.S - c) * vpr;
        for (int v = threadIdx.x; v < nvec; v += kThreads)
            pad[v] = make_uint4(0, 0, 0, 0);
    }
}

// Raster bf16 rows -> per-tile transposed block [D][B]: row f of tile tau
// holds feature f of slots 0..B-1 (empty slots 0).  Rows are gathered with
// 16-byte loads into LDS words [B][D / 2 + 1] (an odd word stride, so the
// column reads below spread over the banks); each output item then reads a
// feature pair of 8 consecutive slots as 8 words and writes two 16-byte
// vectors, one per feature.
template <int D>
__global__ __launch_bounds__(kThreads) void permute_tile_columns_kernel(
    Layout L, const uint16_t *__restrict__ src, uint16_t *__restrict__ dst)
{
    constexpr int LDW = D / 2 + 1;  // words per LDS row
    constexpr int CPR = D / 8;      // 16-byte chunks per row
    __shared__ uint32_t tileW[128 * LDW];
    const int h = blockIdx.x / L.nT;
    const int tau = blockIdx.x - h * L.nT;
    const TileBox bx = tile_box(L, tau);
    const int c = bx.et * bx.ey * bx.ex;
    const int B = L.S;  // slots per tile
    const uint4 *rows = reinterpret_cast<const uint4 *>(src + (long long)h * L.N * D);
    for (int u = threadIdx.x; u < B * CPR; u += kThreads) {
        const int slot = u / CPR, ch = u - slot * CPR;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (slot < c)
            val = rows[(long long)position_token(L, slot_token(L, bx, slot)) * CPR + ch];
        uint32_t *w = tileW + slot * LDW + 4 * ch;
        w[0] = val.x;
        w[1] = val.y;
        w[2] = val.z;
        w[3] = val.w;
    }
    __syncthreads();
    const int groups = B / 8;
    uint16_t *out = dst + ((long long)h * L.nT + tau) * D * B;
    for (int u = threadIdx.x; u < (D / 2) * groups; u += kThreads) {
        const int fp = u / groups, g = u - fp * groups;
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            w[i] = tileW[(8 * g + i) * LDW + fp];
        // Low halves are feature 2 fp, high halves feature 2 fp + 1.
        uint4 lo, hi;
        lo.x = __builtin_amdgcn_perm(w[1], w[0], 0x05040100u);
        lo.y = __builtin_amdgcn_perm(w[3], w[2], 0x05040100u);
        lo.z = __builtin_amdgcn_perm(w[5], w[4], 0x05040100u);
        lo.w = __builtin_amdgcn_perm(w[7], w[6], 0x05040100u);
        hi.x = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u);
        hi.y = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
        hi.z = __builtin_amdgcn_perm(w[5], w[4], 0x07060302u);
        hi.w = __builtin_amdgcn_perm(w[7], w[6], 0x07060302u);
        reinterpret_cast<uint4 *>(out + (long long)(2 * fp) * B)[g] = lo;
        reinterpret_cast<uint4 *>(out + (long long)(2 * fp + 1) * B)[g] = hi;
    }
}

}  // namespace

hipError_t launch_permute_rows(const Layout &L, int elem_bytes, const void *src, void *dst,
                               hipStream_t s)
{
    const int vpr = L.D * elem_bytes / 16;
    hipLaunchKernelGGL(permute_rows_kernel<0>, dim3(L.heads * L.nT), dim3(kThreads), 0, s, L, vpr,
                       (const uint4 *)src, (uint4 *)dst);
    return hipGetLastError();
}

hipError_t launch_unpermute_rows(const Layout &L, int elem_bytes, const void *src, void *dst,
                                 hipStream_t s)
{
    const int vpr = L.D * elem_bytes / 16;
    hipLaunchKernelGGL(permute_rows_kernel<1>, dim3(L.heads * L.nT), dim3(kThreads), 0, s, L, vpr,
                       (const uint4 *)src, (uint4 *)dst);
    return hipGetLastError();
}

hipError_t launch_permute_tile_columns(const Layout &L, const void *src, void *dst, hipStream_t s)
{
    if (L.D == 128)
        hipLaunchKernelGGL(permute_tile_columns_kernel<128>, dim3(L.heads * L.nT), dim3(kThreads), 0,
                           s, L, (const uint16_t *)src, (uint16_t *)dst);
    else
        hipLaunchKernelGGL(permute_tile_columns_kernel<64>, dim3(L.heads * L.nT), dim3(kThreads), 0,
                           s, L, (const uint16_t *)src, (uint16_t *)dst);
    return hipGetLastError();
}

}  // namespace sa
