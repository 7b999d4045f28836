// Reference attention mass per tile pair, for the offline window search.
//
// A[h][i][j] = (1 / c_i) sum over the real queries n of tile i of the
// full-attention softmax mass that n gives the keys of tile j (Compact
// Attention page, Fig. 1 caption: reference attention mass of query-key
// regions; Fig. 4 caption: the search keeps the regions that hold most of a
// head's mass).  Every key takes part, so this is dense work: two passes of
// S = s Q K^T over all key tiles, the first for each query's log-sum-exp,
// the second for exp(s q.k - LSE) summed per key tile.
//
// One workgroup of 8 waves serves two neighbouring query tiles of one head
// (waves 0-3 tile 2r, waves 4-7 tile 2r + 1, 32 queries per wave).  Each key
// tile is staged once in LDS for both (rows padded by 16 bytes, so the 16-byte
// operand reads of 16 consecutive rows hit distinct banks) and read by all 8
// waves as the A operand of v_mfma_f32_32x32x16_bf16 (S^T = K Q^T; Q stays in
// registers as the B operand).  Lane l then holds the scores of query l % 32
// against 16 keys of each 32-key block.  Per key tile, each wave's pass-2
// partial sum goes to LDS and one thread per query tile adds the four.
#include "common.h"

namespace sa {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileRows = 128;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x += __shfl_xor(x, o);
    return x;
}

// Scores S^T of 32 keys (rows kb*32.. of the staged tile) against this
// wave's 32 queries: register r of lane l is key 8 (r / 4) + 4 (l / 32) + r % 4
// of the block, query l % 32.
template <int D>
__device__ __forceinline__ f32x16 block_scores(const char *Ks, int kb, const bf16x8 (&qf)[D / 16],
                                               int l32, int hi)
{
    constexpr int RB = 2 * D + 16;  // padded row bytes
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        acc[r] = 0.f;
    const char *row = Ks + (kb * 32 + l32) * RB + 16 * hi;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = *(const bf16x8 *)(row + 32 * ks);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], acc, 0, 0, 0);
    }
    return acc;
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void mass_kernel(Layout L, const uint16_t *__restrict__ Qt,
                                                           const uint16_t *__restrict__ Kt,
                                                           float scale_log2, float *__restrict__ mass)
{
    constexpr int RB = 2 * D + 16;
    constexpr int KS = D / 16;
    __shared__ __attribute__((aligned(16))) char Ks[kTileRows * RB];
    __shared__ float part[kWaves];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int npairs = (L.nT + 1) / 2;
    const int h = blockIdx.x / npairs;
    const int i0 = 2 * (blockIdx.x - h * npairs);
    const int side = wave >> 2;
    const int i = i0 + side;  // this wave's query tile (may be nT: none)
    const int ci = i < L.nT ? tile_real_count(L, i) : 0;
    const int slot = (wave & 3) * 32 + l32;
    const bool wave_active = (wave & 3) * 32 < ci;
    const bool q_real = slot < ci;

    bf16x8 qf[KS];
    if (wave_active) {
        const bf16x8 *qp =
            (const bf16x8 *)(Qt + ((long long)h * L.Npad + (long long)i * L.B + slot) * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = qp[2 * ks + hi];
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int u = 0; u < 8; ++u)
                qf[ks][u] = (__bf16)0.0f;
    }

    const uint16_t *Kh = Kt + (long long)h * L.Npad * D;
    // Stage key tile j: 128 rows of 2 D bytes as 16-byte pieces (empty slots
    // are zero rows of the permuted K; their scores are masked below).
    auto stage = [&](int j) {
        constexpr int PPR = 2 * D / 16;  // pieces per row
        const uint4 *src = (const uint4 *)(Kh + (long long)j * L.B * D);
        for (int u = tid; u < kTileRows * PPR; u += kThreads) {
            const int rr = u / PPR, pc = u - rr * PPR;
            *(uint4 *)(Ks + rr * RB + 16 * pc) = src[u];
        }
    };

    // Pass 1: running max (log2 units) and sum over every key.
    float m = -INFINITY, l = 0.f;
    for (int j = 0; j < L.nT; ++j) {
        const int cj = tile_real_count(L, j);
        __syncthreads();
        stage(j);
        __syncthreads();
        if (!wave_active)
            continue;
        for (int kb = 0; kb * 32 < cj; ++kb) {
            const f32x16 s = block_scores<D>(Ks, kb, qf, l32, hi);
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb * 32 + 8 * (r / 4) + 4 * hi + r % 4;
                if (key < cj)
                    mx = fmaxf(mx, s[r] * scale_log2);
            }
            const float m_new = fmaxf(m, mx);
            if (m_new > -INFINITY) {
                l *= exp2f(m - m_new);
                m = m_new;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb * 32 + 8 * (r / 4) + 4 * hi + r % 4;
                    if (key < cj)
                        l += exp2f(fmaf(s[r], scale_log2, -m));
                }
            }
        }
    }
    // Lanes l and l ^ 32 hold different keys of the same query.
    const float m_o = __shfl_xor(m, 32), l_o = __shfl_xor(l, 32);
    const float m_all = fmaxf(m, m_o);
    const float l_all = (m > -INFINITY ? l * exp2f(m - m_all) : 0.f) +
                        (m_o > -INFINITY ? l_o * exp2f(m_o - m_all) : 0.f);
    const float lse2 = m_all + log2f(l_all);

    // Pass 2: mass per key tile.
    for (int j = 0; j < L.nT; ++j) {
        const int cj = tile_real_count(L, j);
        __syncthreads();  // the previous tile's partial sums are in part[]
        if (j > 0 && tid < 2 && i0 + tid < L.nT) {
            const int t = i0 + tid;
            const float sum = part[4 * tid] + part[4 * tid + 1] + part[4 * tid + 2] + part[4 * tid + 3];
            mass[((long long)h * L.nT + t) * L.nT + (j - 1)] = sum / (float)tile_real_count(L, t);
        }
        stage(j);
        __syncthreads();
        float acc = 0.f;
        if (wave_active) {
            for (int kb = 0; kb * 32 < cj; ++kb) {
                const f32x16 s = block_scores<D>(Ks, kb, qf, l32, hi);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb * 32 + 8 * (r / 4) + 4 * hi + r % 4;
                    if (key < cj)
                        acc += exp2f(fmaf(s[r], scale_log2, -lse2));
                }
            }
        }
        acc = wave_sum(q_real ? acc : 0.f);
        if (lane == 0)
            part[wave] = acc;
    }
    __syncthreads();
    if (tid < 2 && i0 + tid < L.nT) {
        const int t = i0 + tid;
        const float sum = part[4 * tid] + part[4 * tid + 1] + part[4 * tid + 2] + part[4 * tid + 3];
        mass[((long long)h * L.nT + t) * L.nT + (L.nT - 1)] = sum / (float)tile_real_count(L, t);
    }
}

}  // namespace

hipError_t launch_tile_mass(const Layout &L, const void *q, const void *k, float scale_log2, float *mass,
                            hipStream_t s)
{
    const dim3 grid(L.heads * ((L.nT + 1) / 2));
    if (L.D == 128)
        hipLaunchKernelGGL(mass_kernel<128>, grid, dim3(kThreads), 0, s, L, (const uint16_t *)q,
                           (const uint16_t *)k, scale_log2, mass);
    else
        hipLaunchKernelGGL(mass_kernel<64>, grid, dim3(kThreads), 0, s, L, (const uint16_t *)q,
                           (const uint16_t *)k, scale_log2, mass);
    return hipGetLastError();
}

}  // namespace sa
