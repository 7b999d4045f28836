// Tile selection: a top-k tile mask from Q and K.
//
// The step before the mask compiler when masks are chosen from the inputs
// themselves (SCOPE review page: the abstract names masks built from
// block-level proxy scores, "The reading" a per-head Top-k count, "What
// carries the argument" the 1/sqrt(d) scale of a proxy logit; AdaSpa page,
// abstract: a blockified pattern).  Score of tile pair (i, j) in head h:
// scale * qbar_i . kbar_j, with qbar, kbar the means of the tiles' real
// tokens; row i keeps the k_h tiles with the largest score, ties to the
// lower j.  The output is a tile bitmap for the mask compiler.
//
//   pool   : one workgroup per (head, tile, Q or K): fp32 mean of the tile's
//            real rows of the tile-major Q or K
//   select : one workgroup per (head, 8 query tiles; 1 when nT > 2048): the
//            rows' nT scores into LDS as order-preserving 32-bit keys (each
//            k-bar row read once for the group), then one wave per row: the
//            k-th largest key by a bitwise radix select over the candidates
//            (32 rounds of ballots, most significant bit first), and the
//            row: keys above it, and keys equal to it in increasing j until
//            k are kept (ballot prefix counts).
#include "common.h"

namespace sa {

namespace {

constexpr int kPoolThreads = 256;
constexpr int kSelThreads = 256;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Adds the 8 consecutive elements at p (16-byte aligned) to acc.
__device__ __forceinline__ void add8(float (&acc)[8], const uint16_t *p)
{
    const u32x4 w = *(const u32x4 *)p;  // 8 bf16
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        acc[2 * u] += __uint_as_float(w[u] << 16);
        acc[2 * u + 1] += __uint_as_float(w[u] & 0xffff0000u);
    }
}
__device__ __forceinline__ void add8(float (&acc)[8], const float *p)
{
    const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        acc[u] += a[u];
        acc[4 + u] += b[u];
    }
}

// blockIdx.x = h * nT + tile, blockIdx.y = 0 (Q) / 1 (K).  Thread t sums
// features 8 (t % G) .. + 7 over rows t / G, t / G + RP, ... (G = D / 8
// feature groups, RP = 256 / G rows in flight); the partial sums are then
// reduced through LDS.
template <typename T>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(Layout L, const T *__restrict__ q,
                                                            const T *__restrict__ k,
                                                            float *__restrict__ qbar,
                                                            float *__restrict__ kbar)
{
    __shared__ float part[kPoolThreads * 8];
    const int D = L.D;
    const int G = D / 8, RP = kPoolThreads / G;
    const int ht = blockIdx.x;
    const int h = ht / L.nT, tau = ht - h * L.nT;
    const int c = tile_real_count(L, tau);
    const T *src = (blockIdx.y == 0 ? q : k) + ((long long)h * L.Npad + (long long)tau * L.S) * D;
    float *dst = (blockIdx.y == 0 ? qbar : kbar) + (long long)ht * D;
    const int g = threadIdx.x % G, r0 = threadIdx.x / G;
    float acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
        acc[u] = 0.f;
    for (int r = r0; r < c; r += RP)
        add8(acc, src + (long long)r * D + 8 * g);
#pragma unroll
    for (int u = 0; u < 8; ++u)
        part[threadIdx.x * 8 + u] = acc[u];
    __syncthreads();
    // Feature f = 8 g + u is summed over the RP threads r0 * G + g.
    for (int f = threadIdx.x; f < D; f += kPoolThreads) {
        const int gg = f / 8, u = f % 8;
        float s = 0.f;
        for (int rr = 0; rr < RP; ++rr)
            s += part[(rr * G + gg) * 8 + u];
        dst[f] = c > 0 ? s / (float)c : 0.f;
    }
}

// Order-preserving map of a float to an unsigned key (larger float, larger key).
__device__ __forceinline__ uint32_t sort_key(float x)
{
    const uint32_t b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// blockIdx.x = h * ceil(nT / R) + g: query tiles i = g R .. g R + R - 1 of
// head h.  Each k-bar row is read once for the R query tiles (their q-bar
// rows wait in LDS), so the k-bar traffic is 1 / R of one row per group.
// keys: dynamic LDS [R][nT].
template <int R>
__global__ __launch_bounds__(kSelThreads) void select_kernel(Layout L, const float *__restrict__ qbar,
                                                             const float *__restrict__ kbar,
                                                             const int *__restrict__ kh, float scale,
                                                             uint8_t *__restrict__ bitmap)
{
    extern __shared__ uint32_t keys[];
    __shared__ float qi[R][128];
    const int nT = L.nT, D = L.D;
    const int ngroups = (nT + R - 1) / R;
    const int h = blockIdx.x / ngroups;
    const int i0 = (blockIdx.x - h * ngroups) * R;
    const int rows = min(R, nT - i0);
    const int tid = threadIdx.x;
    const int kk = kh[h];
    if (kk <= 0 || kk >= nT) {
        for (int u = tid; u < rows * nT; u += kSelThreads)
            bitmap[((long long)h * nT + i0) * nT + u] = kk > 0 ? 1 : 0;
        return;
    }
    for (int u = tid; u < R * D; u += kSelThreads) {
        const int r = u / D, e = u - r * D;
        qi[r][e] = r < rows ? qbar[((long long)h * nT + i0 + r) * D + e] : 0.f;
    }
    __syncthreads();
    const float *kb = kbar + (long long)h * nT * D;
    for (int j = tid; j < nT; j += kSelThreads) {
        const float4 *kr = (const float4 *)(kb + (long long)j * D);
        float dot[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            dot[r] = 0.f;
        for (int e4 = 0; e4 < D / 4; ++e4) {
            const float4 v = kr[e4];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                dot[r] = fmaf(qi[r][4 * e4], v.x, dot[r]);
                dot[r] = fmaf(qi[r][4 * e4 + 1], v.y, dot[r]);
                dot[r] = fmaf(qi[r][4 * e4 + 2], v.z, dot[r]);
                dot[r] = fmaf(qi[r][4 * e4 + 3], v.w, dot[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            keys[r * nT + j] = sort_key(dot[r] * scale);
    }
    __syncthreads();
    // One wave per row: the k-th largest key by a bitwise radix select with
    // ballots (candidates = keys matching the bits fixed so far), then the
    // row.  Key j sits in lane j % 64 of slot j / 64.
    const int lane = tid & 63, wave = tid >> 6;
    const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int slots = (nT + 63) / 64;
    for (int r = wave; r < rows; r += kSelThreads / 64) {
        const uint32_t *rk = keys + r * nT;
        uint32_t prefix = 0, fixed = 0;  // value and mask of the bits fixed so far
        int remaining = kk;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t b = 1u << bit;
            int ones = 0;
            for (int sl = 0; sl < slots; ++sl) {
                const int j = sl * 64 + lane;
                const uint32_t key = j < nT ? rk[j] : 0u;
                const bool cand = j < nT && (key & fixed) == prefix;
                ones += __popcll(__ballot(cand && (key & b)));
            }
            if (ones >= remaining)
                prefix |= b;
            else
                remaining -= ones;
            fixed |= b;
        }
        // prefix is the k-th largest key; keep the keys above it and the
        // first `remaining` keys equal to it in increasing j.
        uint8_t *out = bitmap + ((long long)h * nT + i0 + r) * nT;
        int taken_eq = 0;
        for (int sl = 0; sl < slots; ++sl) {
            const int j = sl * 64 + lane;
            const uint32_t key = j < nT ? rk[j] : 0u;
            const bool eq = j < nT && key == prefix;
            const unsigned long long eqs = __ballot(eq);
            const int rank = taken_eq + __popcll(eqs & below);
            if (j < nT)
                out[j] = (key > prefix || (eq && rank < remaining)) ? 1 : 0;
            taken_eq += __popcll(eqs);
        }
    }
}

}  // namespace

hipError_t launch_select_topk(const Layout &L, int elem_bytes, const void *q, const void *k,
                              const int *kh, float scale, float *qbar, float *kbar, uint8_t *bitmap,
                              hipStream_t s)
{
    const dim3 pool_grid(L.heads * L.nT, 2);
    if (elem_bytes == 2)
        hipLaunchKernelGGL(pool_kernel<uint16_t>, pool_grid, dim3(kPoolThreads), 0, s, L,
                           (const uint16_t *)q, (const uint16_t *)k, qbar, kbar);
    else
        hipLaunchKernelGGL(pool_kernel<float>, pool_grid, dim3(kPoolThreads), 0, s, L, (const float *)q,
                           (const float *)k, qbar, kbar);
    // R query tiles per workgroup, their keys in LDS (at most 64 KB).
    constexpr int R = 8;
    if ((size_t)R * L.nT * sizeof(uint32_t) <= 65536) {
        const dim3 grid(L.heads * ((L.nT + R - 1) / R));
        hipLaunchKernelGGL(select_kernel<R>, grid, dim3(kSelThreads), sizeof(uint32_t) * (size_t)R * L.nT, s, L,
                           qbar, kbar, kh, scale, bitmap);
    } else {
        hipLaunchKernelGGL(select_kernel<1>, dim3(L.heads * L.nT), dim3(kSelThreads),
                           sizeof(uint32_t) * (size_t)L.nT, s, L, qbar, kbar, kh, scale, bitmap);
    }
    return hipGetLastError();
}

}  // namespace sa
