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
//   select : one workgroup per (head, query tile): the row's nT scores into
//            LDS as order-preserving 32-bit keys, the k-th largest key by a
//            4-pass radix select (8 bits per pass, most significant first),
//            then the row: keys above it, and keys equal to it in increasing
//            j until k are kept (a workgroup-wide prefix count over j).
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
    const T *src = (blockIdx.y == 0 ? q : k) + ((long long)h * L.Npad + (long long)tau * L.B) * D;
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

// Exclusive prefix count of `flag` over the workgroup's threads (in thread
// order); returns the count before this thread, *total the workgroup's count.
__device__ __forceinline__ int block_prefix_count(bool flag, int *wave_cnt, int *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned long long bits = __ballot(flag);
    const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int in_wave = __popcll(bits & below);
    __syncthreads();  // wave_cnt is free again
    if (lane == 0)
        wave_cnt[wave] = __popcll(bits);
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) {
        before += w < wave ? wave_cnt[w] : 0;
        all += wave_cnt[w];
    }
    *total = all;
    return before + in_wave;
}

// blockIdx.x = h * nT + i.  keys: dynamic LDS of nT entries.
__global__ __launch_bounds__(kSelThreads) void select_kernel(Layout L, const float *__restrict__ qbar,
                                                             const float *__restrict__ kbar,
                                                             const int *__restrict__ kh, float scale,
                                                             uint8_t *__restrict__ bitmap)
{
    extern __shared__ uint32_t keys[];
    __shared__ float qi[128];
    __shared__ int hist[256];
    __shared__ int wave_cnt[kSelThreads / 64];
    __shared__ uint32_t sel[2];  // prefix digit found by a pass, remaining count
    const int nT = L.nT, D = L.D;
    const int hi = blockIdx.x;
    const int h = hi / nT;
    const int tid = threadIdx.x;
    const int kk = kh[h];
    uint8_t *out = bitmap + (long long)hi * nT;
    if (kk <= 0 || kk >= nT) {
        for (int j = tid; j < nT; j += kSelThreads)
            out[j] = kk > 0 ? 1 : 0;
        return;
    }
    for (int e = tid; e < D; e += kSelThreads)
        qi[e] = qbar[(long long)hi * D + e];
    __syncthreads();
    const float *kb = kbar + (long long)h * nT * D;
    for (int j = tid; j < nT; j += kSelThreads) {
        const float4 *kr = (const float4 *)(kb + (long long)j * D);
        float dot = 0.f;
        for (int e4 = 0; e4 < D / 4; ++e4) {
            const float4 v = kr[e4];
            dot = fmaf(qi[4 * e4], v.x, dot);
            dot = fmaf(qi[4 * e4 + 1], v.y, dot);
            dot = fmaf(qi[4 * e4 + 2], v.z, dot);
            dot = fmaf(qi[4 * e4 + 3], v.w, dot);
        }
        keys[j] = sort_key(dot * scale);
    }
    // Radix select of the kk-th largest key.
    uint32_t prefix = 0, pmask = 0;
    int remaining = kk;
    for (int pass = 3; pass >= 0; --pass) {
        const int shift = 8 * pass;
        for (int b = tid; b < 256; b += kSelThreads)
            hist[b] = 0;
        __syncthreads();
        for (int j = tid; j < nT; j += kSelThreads) {
            const uint32_t key = keys[j];
            if ((key & pmask) == prefix)
                atomicAdd(&hist[(key >> shift) & 255], 1);
        }
        __syncthreads();
        if (tid == 0) {
            int above = 0, b = 255;
            for (; b > 0; --b) {
                if (above + hist[b] >= remaining)
                    break;
                above += hist[b];
            }
            sel[0] = (uint32_t)b;
            sel[1] = (uint32_t)(remaining - above);
        }
        __syncthreads();
        prefix |= sel[0] << shift;
        pmask |= 255u << shift;
        remaining = (int)sel[1];
        __syncthreads();  // sel is rewritten by the next pass
    }
    // Keep keys above the threshold, and the first `remaining` equal ones.
    int taken_eq = 0;
    for (int j0 = 0; j0 < nT; j0 += kSelThreads) {
        const int j = j0 + tid;
        const uint32_t key = j < nT ? keys[j] : 0u;
        const bool eq = j < nT && key == prefix;
        int total;
        const int rank = taken_eq + block_prefix_count(eq, wave_cnt, &total);
        if (j < nT)
            out[j] = (key > prefix || (eq && rank < remaining)) ? 1 : 0;
        taken_eq += total;
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
    const size_t lds = sizeof(uint32_t) * (size_t)L.nT;
    hipLaunchKernelGGL(select_kernel, dim3(L.heads * L.nT), dim3(kSelThreads), lds, s, L, qbar, kbar, kh,
                       scale, bitmap);
    return hipGetLastError();
}

}  // namespace sa
