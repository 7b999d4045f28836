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

// Value of an order-preserving key (inverse of sort_key).
__device__ __forceinline__ float key_value(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x += __shfl_xor(x, o);
    return x;
}

// Scores of query tiles i0 .. i0 + rows - 1 of head h against every key
// tile, as order-preserving keys in keys[r * nT + j].  Each k-bar row is
// read once for the R query tiles (their q-bar rows wait in qi), so the
// k-bar traffic is 1 / R of one row per group.
template <int R>
__device__ __forceinline__ void row_keys(const Layout &L, const float *__restrict__ qbar,
                                         const float *__restrict__ kbar, float scale, int h, int i0, int rows,
                                         uint32_t *keys, float (&qi)[R][128])
{
    const int nT = L.nT, D = L.D, tid = threadIdx.x;
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
}

// blockIdx.x = h * ceil(nT / R) + g: query tiles i = g R .. g R + R - 1 of
// head h; row i keeps its k best-scoring key tiles, k = kn[h] (per_row = 0)
// or kn[h nT + i] (per_row = 1).  keys: dynamic LDS [R][nT].
template <int R>
__global__ __launch_bounds__(kSelThreads) void select_kernel(Layout L, const float *__restrict__ qbar,
                                                             const float *__restrict__ kbar,
                                                             const int *__restrict__ kn, int per_row, float scale,
                                                             uint8_t *__restrict__ bitmap)
{
    extern __shared__ uint32_t keys[];
    __shared__ float qi[R][128];
    const int nT = L.nT;
    const int ngroups = (nT + R - 1) / R;
    const int h = blockIdx.x / ngroups;
    const int i0 = (blockIdx.x - h * ngroups) * R;
    const int rows = min(R, nT - i0);
    const int tid = threadIdx.x;
    auto k_of = [&](int r) { return per_row ? kn[h * nT + i0 + r] : kn[h]; };
    // Rows that keep no tile or every tile need no scores.
    bool scored = false;
    for (int r = 0; r < rows; ++r)
        scored |= k_of(r) > 0 && k_of(r) < nT;
    if (!scored) {
        for (int u = tid; u < rows * nT; u += kSelThreads)
            bitmap[((long long)h * nT + i0) * nT + u] = k_of(u / nT) > 0 ? 1 : 0;
        return;
    }
    row_keys<R>(L, qbar, kbar, scale, h, i0, rows, keys, qi);
    // One wave per row: the k-th largest key by a bitwise radix select with
    // ballots (candidates = keys matching the bits fixed so far), then the
    // row.  Key j sits in lane j % 64 of slot j / 64.
    const int lane = tid & 63, wave = tid >> 6;
    const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int slots = (nT + 63) / 64;
    for (int r = wave; r < rows; r += kSelThreads / 64) {
        const uint32_t *rk = keys + r * nT;
        uint8_t *out = bitmap + ((long long)h * nT + i0 + r) * nT;
        const int kk = k_of(r);
        if (kk <= 0 || kk >= nT) {
            for (int j = lane; j < nT; j += 64)
                out[j] = kk > 0 ? 1 : 0;
            continue;
        }
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

// Base counts of the per-head Top-k estimate (SCOPE review page, "What
// carries the argument": a hybrid Top-p / fixed Top-k count per query
// cluster), one query tile per row: p_i = the smallest m such that the m
// largest softmax probabilities of the row's scores sum to at least rho
// (0 for rho <= 0, nT for rho >= 1); base[h nT + i] = min(nT, max(p_i, k_fixed)).
// Dynamic LDS: keys [R][nT], then the unnormalized probabilities [R][nT].
//
// One wave per row: the row maximum, e_j = exp(s_j - max) and Z = sum e_j;
// then the largest key T with mass(keys >= T) >= rho Z by a bitwise search
// (32 rounds of masked wave sums, most significant bit first); p = (keys
// above T) + the number of keys equal to T needed to cover the rest,
// ceil((rho Z - mass(keys > T)) / e_T), clamped to [1, ties].
template <int R>
__global__ __launch_bounds__(kSelThreads) void scope_base_kernel(Layout L, const float *__restrict__ qbar,
                                                                 const float *__restrict__ kbar, float scale,
                                                                 float rho, int k_fixed, int *__restrict__ base)
{
    extern __shared__ uint32_t keys[];
    __shared__ float qi[R][128];
    const int nT = L.nT;
    const int ngroups = (nT + R - 1) / R;
    const int h = blockIdx.x / ngroups;
    const int i0 = (blockIdx.x - h * ngroups) * R;
    const int rows = min(R, nT - i0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (!(rho > 0.f && rho < 1.f)) {
        const int p = rho > 0.f ? nT : 0;
        for (int r = tid; r < rows; r += kSelThreads)
            base[h * nT + i0 + r] = min(nT, max(p, k_fixed));
        return;
    }
    row_keys<R>(L, qbar, kbar, scale, h, i0, rows, keys, qi);
    float *evals = reinterpret_cast<float *>(keys + R * nT);
    const int slots = (nT + 63) / 64;
    constexpr float kLog2e = 1.4426950408889634f;
    for (int r = wave; r < rows; r += kSelThreads / 64) {
        const uint32_t *rk = keys + r * nT;
        float *re = evals + r * nT;
        uint32_t mk = 0;
        for (int j = lane; j < nT; j += 64)
            mk = max(mk, rk[j]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            mk = max(mk, (uint32_t)__shfl_xor((int)mk, o));
        const float smax = key_value(mk);
        float z = 0.f;
        for (int j = lane; j < nT; j += 64) {
            const float e = __builtin_amdgcn_exp2f((key_value(rk[j]) - smax) * kLog2e);
            re[j] = e;
            z += e;
        }
        const float target = rho * wave_sum(z);
        auto mass_from = [&](uint32_t lo, bool strict) {
            float m = 0.f;
            for (int sl = 0; sl < slots; ++sl) {
                const int j = sl * 64 + lane;
                if (j < nT && (strict ? rk[j] > lo : rk[j] >= lo))
                    m += re[j];
            }
            return wave_sum(m);
        };
        uint32_t T = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t c = T | (1u << bit);
            if (mass_from(c, false) >= target)
                T = c;
        }
        int above = 0, ties = 0;
        float eT = 0.f;
        for (int sl = 0; sl < slots; ++sl) {
            const int j = sl * 64 + lane;
            const bool in = j < nT;
            above += __popcll(__ballot(in && rk[j] > T));
            const unsigned long long eq = __ballot(in && rk[j] == T);
            ties += __popcll(eq);
            if (eq && eT == 0.f)
                eT = re[sl * 64 + __ffsll((long long)eq) - 1];
        }
        const float need = target - mass_from(T, true);
        int extra = 0;
        if (ties > 0) {
            const float q = eT > 0.f ? need / eT : (float)ties;
            extra = q <= 1.f ? 1 : (q >= (float)ties ? ties : (int)ceilf(q));
        }
        if (lane == 0)
            base[h * nT + i0 + r] = min(nT, max(above + extra, k_fixed));
    }
}

// Per-head estimate and final counts (SCOPE review page, "What carries the
// argument", Eqs. 9 and 10): k_head = ceil(sum_i c_i base_i / sum_i c_i),
// c_i the real tokens of query tile i (the sum is the head's N); keep_i =
// max(base_i, k_head).  One workgroup per head; exact integer arithmetic.
__global__ __launch_bounds__(kSelThreads) void scope_keep_kernel(Layout L, const int *__restrict__ base,
                                                                 int *__restrict__ keep)
{
    __shared__ unsigned long long part[kSelThreads];
    const int h = blockIdx.x, nT = L.nT, tid = threadIdx.x;
    unsigned long long s = 0;
    for (int i = tid; i < nT; i += kSelThreads)
        s += (unsigned long long)tile_real_count(L, i) * (unsigned long long)base[h * nT + i];
    part[tid] = s;
    __syncthreads();
    for (int w = kSelThreads / 2; w > 0; w >>= 1) {
        if (tid < w)
            part[tid] += part[tid + w];
        __syncthreads();
    }
    const unsigned long long n = (unsigned long long)L.N;
    const int kh = (int)((part[0] + n - 1) / n);
    for (int i = tid; i < nT; i += kSelThreads)
        keep[h * nT + i] = max(base[h * nT + i], kh);
}

// Pooling of Q and K into tile means.
void launch_pool(const Layout &L, int elem_bytes, const void *q, const void *k, float *qbar, float *kbar,
                        hipStream_t s)
{
    const dim3 pool_grid(L.heads * L.nT, 2);
    if (elem_bytes == 2)
        hipLaunchKernelGGL(pool_kernel<uint16_t>, pool_grid, dim3(kPoolThreads), 0, s, L,
                           (const uint16_t *)q, (const uint16_t *)k, qbar, kbar);
    else
        hipLaunchKernelGGL(pool_kernel<float>, pool_grid, dim3(kPoolThreads), 0, s, L, (const float *)q,
                           (const float *)k, qbar, kbar);
}

// Rows per workgroup of the row kernels: R query tiles with `per_row` 32-bit
// LDS words per score, at most 64 KB.
int rows_per_group(const Layout &L, int words)
{
    return (size_t)8 * L.nT * words * sizeof(uint32_t) <= 65536 ? 8 : 1;
}

void launch_select_rows(const Layout &L, const float *qbar, const float *kbar, const int *kn, int per_row,
                               float scale, uint8_t *bitmap, hipStream_t s)
{
    if (rows_per_group(L, 1) == 8)
        hipLaunchKernelGGL(select_kernel<8>, dim3(L.heads * ((L.nT + 7) / 8)), dim3(kSelThreads),
                           sizeof(uint32_t) * (size_t)8 * L.nT, s, L, qbar, kbar, kn, per_row, scale, bitmap);
    else
        hipLaunchKernelGGL(select_kernel<1>, dim3(L.heads * L.nT), dim3(kSelThreads),
                           sizeof(uint32_t) * (size_t)L.nT, s, L, qbar, kbar, kn, per_row, scale, bitmap);
}

}  // namespace

hipError_t launch_select_topk(const Layout &L, int elem_bytes, const void *q, const void *k,
                              const int *kh, float scale, float *qbar, float *kbar, uint8_t *bitmap,
                              hipStream_t s)
{
    launch_pool(L, elem_bytes, q, k, qbar, kbar, s);
    launch_select_rows(L, qbar, kbar, kh, 0, scale, bitmap, s);
    return hipGetLastError();
}

hipError_t launch_select_scope(const Layout &L, int elem_bytes, const void *q, const void *k, float scale,
                               float rho, int k_fixed, float *qbar, float *kbar, int *base, int *keep,
                               uint8_t *bitmap, hipStream_t s)
{
    launch_pool(L, elem_bytes, q, k, qbar, kbar, s);
    if (rows_per_group(L, 2) == 8)
        hipLaunchKernelGGL(scope_base_kernel<8>, dim3(L.heads * ((L.nT + 7) / 8)), dim3(kSelThreads),
                           2 * sizeof(uint32_t) * (size_t)8 * L.nT, s, L, qbar, kbar, scale, rho, k_fixed, base);
    else
        hipLaunchKernelGGL(scope_base_kernel<1>, dim3(L.heads * L.nT), dim3(kSelThreads),
                           2 * sizeof(uint32_t) * (size_t)L.nT, s, L, qbar, kbar, scale, rho, k_fixed, base);
    hipLaunchKernelGGL(scope_keep_kernel, dim3(L.heads), dim3(kSelThreads), 0, s, L, base, keep);
    launch_select_rows(L, qbar, kbar, keep, 1, scale, bitmap, s);
    return hipGetLastError();
}

}  // namespace sa
