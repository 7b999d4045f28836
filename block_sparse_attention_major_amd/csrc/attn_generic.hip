// Block-sparse attention forward on the vector ALUs, fp32 arithmetic
// throughout (fp32 or bf16 inputs).  Serves any tile volume up to 128 and
// head_dim 64 or 128, in particular the fp32 path, where probabilities stay
// in fp32 end to end.  Same semantics as the matrix-core kernel: exact
// softmax attention over the keys of the kept key tiles, zero for a query
// tile that keeps nothing.
//
// One workgroup of 256 threads per (head, query tile); two threads per query
// slot, each owning half of the features (partial dot products are combined
// with the neighbouring lane).  Keys pass through LDS 64 at a time and are
// processed 16 at a time with an online softmax.  Q and O rows go to the
// caller's raster tensors or the tile-major workspace, and the log-sum-exp
// is written on request.
#include "common.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ void store_as(float *p, float x) { *p = x; }
__device__ __forceinline__ void store_as(uint16_t *p, float x)
{
    const __bf16 b = (__bf16)x;
    *p = *reinterpret_cast<const uint16_t *>(&b);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attn_generic_kernel(Layout L, AttnParams P)
{
    constexpr int DH = D / 2;
    __shared__ float Ks[kChunk][D];
    __shared__ float Vs[kChunk][D];
    const T *__restrict__ Qp = (const T *)P.q;
    const T *__restrict__ Kp = (const T *)P.k;
    const T *__restrict__ Vp = (const T *)P.v;
    T *__restrict__ Op = (T *)P.o;

    const int tid = threadIdx.x;
    const int slot = tid >> 1, part = tid & 1;
    const int r = P.rows.order[blockIdx.x];
    const int h = r / L.nT, i = r - h * L.nT;
    const int ci = tile_real_count(L, i);
    const bool active = slot < L.S && slot < ci;
    const float sl2 = P.scale_log2;

    // Row of this slot's query in q and o: the raster token (raster I/O) or
    // the tile-major slot.
    const int tok = (active && (P.raster || P.lse)) ? raster_token(L, i, slot) : 0;
    const long long qrow = P.raster ? (long long)h * L.N + tok : (long long)h * L.Npad + (long long)i * L.S + slot;
    float q[DH], o[DH];
#pragma unroll
    for (int e = 0; e < DH; ++e) {
        q[e] = active ? to_f32(Qp[qrow * D + part * DH + e]) * sl2 : 0.f;
        o[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    const int beg = P.rows.row_ptr[r];
    const int end = (int)min((long long)P.rows.row_ptr[r + 1], P.rows.cap);
    for (int idx = beg; idx < end; ++idx) {
        const int j = P.rows.cols[idx];
        const int cj = tile_real_count(L, j);
        const long long krow0 = (long long)h * L.Npad + (long long)j * L.S;
        for (int k0 = 0; k0 < cj; k0 += kChunk) {
            const int kn = min(kChunk, cj - k0);
            __syncthreads();
            for (int u = tid; u < kn * D; u += kThreads) {
                const int kk = u / D, e = u - kk * D;
                Ks[kk][e] = to_f32(Kp[(krow0 + k0 + kk) * D + e]);
                Vs[kk][e] = to_f32(Vp[(krow0 + k0 + kk) * D + e]);
            }
            __syncthreads();
            if (!active)
                continue;
            for (int kk0 = 0; kk0 < kn; kk0 += 16) {
                float s[16];
                float mx = -INFINITY;
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    float dot = 0.f;
                    if (kk0 + u < kn) {
#pragma unroll
                        for (int e = 0; e < DH; ++e)
                            dot = fmaf(q[e], Ks[kk0 + u][part * DH + e], dot);
                    }
                    dot += __shfl_xor(dot, 1);
                    s[u] = kk0 + u < kn ? dot : -INFINITY;
                    mx = fmaxf(mx, s[u]);
                }
                const float m_new = fmaxf(m, mx);
                const float alpha = __builtin_amdgcn_exp2f(m - m_new);
                l *= alpha;
#pragma unroll
                for (int e = 0; e < DH; ++e)
                    o[e] *= alpha;
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const float p = __builtin_amdgcn_exp2f(s[u] - m_new);
                    l += p;
                    if (kk0 + u < kn) {
#pragma unroll
                        for (int e = 0; e < DH; ++e)
                            o[e] = fmaf(p, Vs[kk0 + u][part * DH + e], o[e]);
                    }
                }
                m = m_new;
            }
        }
    }
    if (active) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        // m is in log2 units (q carries scale * log2 e) and l sums exp2(s - m).
        if (P.lse && part == 0)
            P.lse[(long long)h * L.N + tok] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
#pragma unroll
        for (int e = 0; e < DH; ++e)
            store_as(&Op[qrow * D + part * DH + e], o[e] * inv);
    }
}

template <typename T>
hipError_t launch_typed(const Layout &L, const AttnParams &p, hipStream_t s)
{
    const dim3 grid(L.heads * L.nT);
    if (L.D == 128)
        hipLaunchKernelGGL((attn_generic_kernel<T, 128>), grid, dim3(kThreads), 0, s, L, p);
    else
        hipLaunchKernelGGL((attn_generic_kernel<T, 64>), grid, dim3(kThreads), 0, s, L, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_generic(const Layout &L, int elem_bytes, const AttnParams &p,
                                    hipStream_t s)
{
    return elem_bytes == 4 ? launch_typed<float>(L, p, s) : launch_typed<uint16_t>(L, p, s);
}

}  // namespace sa
