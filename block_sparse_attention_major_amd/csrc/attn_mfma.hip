// Block-sparse flash attention forward, bf16 in / fp32 accumulate, on the
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// What is computed: for every query tile i of head h, exact softmax
// attention over the keys of the key tiles its mask row keeps (Compact
// Attention page, Fig. 3 caption: precomputed masks run in block-sparse
// attention kernels; SCOPE review page, abstract: attention over the selected
// original keys and values).  Dropped tile pairs cost no loads and no FLOPs.
//
// Design (ours, for CDNA4; the pages give no kernel design):
//  - One workgroup of 4 waves per (head, query tile); tile = 128 slots, each
//    wave owns 32 query slots.  Workgroups run in the compiled longest-first
//    order.
//  - Keys are consumed in stages of 64 (half a tile); a stage of K and of the
//    transposed V tile is staged in LDS, double-buffered, so the next stage's
//    global loads overlap this stage's math.  The empty tail of a clipped
//    key tile (80 of 128 slots at 720p) is skipped at 32-key granularity.
//  - Scores are computed transposed, S^T = K Q^T, so each lane holds 16 keys
//    of one query: row max and row sum are in-lane, plus one exchange with
//    the lane 32 apart.  K rows are fed to the MFMA in a permuted order so the
//    probabilities come out already in the operand order of the next MFMA,
//    O^T += V^T P^T, whose accumulator again keeps one query per lane (the
//    rescale by exp(m_old - m_new) is in-lane).
//  - V arrives pre-transposed per tile ([D][128], written by the permute
//    stage), so V^T operand reads are plain 16-byte LDS reads.
//  - LDS rows are XOR-swizzled in 16-byte chunks so the MFMA operand reads and
//    the staging writes are free of bank conflicts.
//  - Online softmax in fp32 with exp2 and the scale folded into one FMA.
#include "common.h"

namespace sa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTile = 128;   // slots per tile
constexpr int kStage = 64;   // keys per LDS stage

// Byte offset of 16-byte chunk c of row `row` in an LDS block whose rows hold
// RC chunks.  Rows are packed into 256-byte lines; the chunk index is XORed
// with the line index so 16 consecutive rows read at one column hit 16
// different chunk positions.
template <int RC>
__device__ __forceinline__ int lds_off(int row, int c)
{
    constexpr int RPL = 16 / RC;
    const int line = row / RPL;
    const int logical = (row % RPL) * RC + c;
    return line * 256 + ((logical ^ (line & 15)) << 4);
}

// Key row fed to MFMA row m of a 32-key subtile.  With this order, result
// register j of lane l holds key 16 (j / 8) + 8 (l / 32) + j % 8, which is
// the B-operand order of the P V^T product.
__device__ __forceinline__ int key_of_mfma_row(int m)
{
    const int a = m >> 3, b = (m >> 2) & 1, c = m & 3;
    return 16 * (a >> 1) + 8 * b + 4 * (a & 1) + c;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-thread share of one stage: K rows [64][D] and transposed V [D][64].
template <int D>
struct StageShape {
    static constexpr int RCK = D / 8;                    // 16-byte chunks per K row
    static constexpr int KPT = kStage * RCK / kThreads;  // K chunks per thread
    static constexpr int VPT = D * 8 / kThreads;         // V chunks per thread
    static constexpr int K_BYTES = kStage * D * 2;
    static constexpr int BYTES = 2 * K_BYTES;
};

// Global -> registers: 64 keys (half `half` of key tile j) of K and of the
// transposed V tile.
template <int D>
__device__ __forceinline__ void load_stage(u32x4 (&stK)[StageShape<D>::KPT],
                                           u32x4 (&stV)[StageShape<D>::VPT],
                                           const uint16_t *__restrict__ Kp,
                                           const uint16_t *__restrict__ Vt, const Layout &L, int h,
                                           int j, int half, int tid)
{
    using S = StageShape<D>;
    const uint16_t *kb = Kp + ((long long)h * L.Npad + (long long)j * kTile + half * kStage) * D;
    const uint16_t *vb = Vt + ((long long)h * L.nT + j) * D * kTile + half * kStage;
#pragma unroll
    for (int t = 0; t < S::KPT; ++t) {
        const int u = tid + kThreads * t, row = u / S::RCK, c = u % S::RCK;
        stK[t] = *(const u32x4 *)(kb + row * D + 8 * c);
    }
#pragma unroll
    for (int t = 0; t < S::VPT; ++t) {
        const int u = tid + kThreads * t, row = u >> 3, c = u & 7;
        stV[t] = *(const u32x4 *)(vb + (long long)row * kTile + 8 * c);
    }
}

// Registers -> one LDS stage buffer, swizzled.
template <int D>
__device__ __forceinline__ void store_stage(const u32x4 (&stK)[StageShape<D>::KPT],
                                            const u32x4 (&stV)[StageShape<D>::VPT], char *base,
                                            int tid)
{
    using S = StageShape<D>;
#pragma unroll
    for (int t = 0; t < S::KPT; ++t) {
        const int u = tid + kThreads * t, row = u / S::RCK, c = u % S::RCK;
        *(u32x4 *)(base + lds_off<S::RCK>(row, c)) = stK[t];
    }
#pragma unroll
    for (int t = 0; t < S::VPT; ++t) {
        const int u = tid + kThreads * t, row = u >> 3, c = u & 7;
        *(u32x4 *)(base + S::K_BYTES + lds_off<8>(row, c)) = stV[t];
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_mfma_kernel(Layout L, AttnParams P)
{
    constexpr int KS = D / 16;                 // QK^T k-steps
    constexpr int NB = D / 32;                 // 32-wide feature blocks of O^T
    constexpr int RCK = D / 8;                 // 16-byte chunks per K row
    constexpr int K_BYTES = kStage * D * 2;
    constexpr int V_BYTES = D * kStage * 2;
    constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
    constexpr int KPT = kStage * RCK / kThreads;  // K chunks per thread per stage
    constexpr int VPT = D * 8 / kThreads;         // V chunks per thread per stage
    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];

    const uint16_t *__restrict__ Qp = (const uint16_t *)P.q;
    const uint16_t *__restrict__ Kp = (const uint16_t *)P.k;
    const uint16_t *__restrict__ Vt = (const uint16_t *)P.v;
    uint16_t *__restrict__ Op = (uint16_t *)P.o;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hi = lane >> 5;
    const int r = P.order[blockIdx.x];
    const int h = r / L.nT, i = r - h * L.nT;
    const int ci = tile_real_count(L, i);
    const bool wave_active = wave * 32 < ci;

    // Q operand (B of S^T = K Q^T): lane holds query l32, features
    // 16 ks + 8 hi .. +7 for every k-step.
    const long long qrow = (long long)h * L.Npad + (long long)i * kTile + wave * 32 + l32;
    bf16x8 qf[KS];
    {
        const bf16x8 *qp = (const bf16x8 *)(Qp + qrow * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = qp[2 * ks + hi];
    }

    f32x16 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            acc[nb][jj] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = P.scale_log2;

    const int beg = P.row_ptr[r];
    const int end = (int)min((long long)P.row_ptr[r + 1], P.cap);

    u32x4 stK[KPT], stV[VPT];
    int idx = beg, half = 0, buf = 0;
    if (idx < end) {
        load_stage<D>(stK, stV, Kp, Vt, L, h, P.cols[idx], half, tid);
        store_stage<D>(stK, stV, smem, tid);
    }
    const int prow = key_of_mfma_row(l32);
    while (idx < end) {
        const int cj = tile_real_count(L, P.cols[idx]);
        const int kv = min(kStage, cj - half * kStage);  // real keys in this stage
        int nidx = idx, nhalf = half + 1;
        if (nhalf * kStage >= cj) {
            ++nidx;
            nhalf = 0;
        }
        const bool more = nidx < end;
        __syncthreads();  // stage `buf` is complete; the other buffer is free
        if (more)
            load_stage<D>(stK, stV, Kp, Vt, L, h, P.cols[nidx], nhalf, tid);

        if (wave_active) {
            const char *Ks = smem + buf * STAGE_BYTES;
            const char *Vs = Ks + K_BYTES;
            const bool two = kv > 32;
            f32x16 s0, s1;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                s0[jj] = 0.f;
                s1[jj] = 0.f;
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    *(const bf16x8 *)(Ks + lds_off<RCK>(prow, 2 * ks + hi)), qf[ks], s0, 0, 0, 0);
            if (two) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        *(const bf16x8 *)(Ks + lds_off<RCK>(32 + prow, 2 * ks + hi)), qf[ks], s1, 0,
                        0, 0);
            }
            if (kv < kStage) {
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    const int key = 16 * (jj >> 3) + 8 * hi + (jj & 7);
                    if (key >= kv)
                        s0[jj] = -INFINITY;
                    if (32 + key >= kv)
                        s1[jj] = -INFINITY;
                }
            }
            float mx = s0[0];
#pragma unroll
            for (int jj = 1; jj < 16; ++jj)
                mx = fmaxf(mx, s0[jj]);
            if (two) {
#pragma unroll
                for (int jj = 0; jj < 16; ++jj)
                    mx = fmaxf(mx, s1[jj]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float alpha = exp2_fast((m_run - m_new) * sl2);
            const float mb = m_new * sl2;
            float psum = 0.f;
            bf16x8 p0a, p0b, p1a, p1b;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const float e0 = exp2_fast(fmaf(s0[jj], sl2, -mb));
                const float e1 = exp2_fast(fmaf(s0[jj + 8], sl2, -mb));
                psum += e0 + e1;
                p0a[jj] = (__bf16)e0;
                p0b[jj] = (__bf16)e1;
            }
            if (two) {
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const float e0 = exp2_fast(fmaf(s1[jj], sl2, -mb));
                    const float e1 = exp2_fast(fmaf(s1[jj + 8], sl2, -mb));
                    psum += e0 + e1;
                    p1a[jj] = (__bf16)e0;
                    p1b[jj] = (__bf16)e1;
                }
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int jj = 0; jj < 16; ++jj)
                    acc[nb][jj] *= alpha;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int vrow = 32 * nb + l32;
                acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    *(const bf16x8 *)(Vs + lds_off<8>(vrow, 0 + hi)), p0a, acc[nb], 0, 0, 0);
                acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    *(const bf16x8 *)(Vs + lds_off<8>(vrow, 2 + hi)), p0b, acc[nb], 0, 0, 0);
                if (two) {
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        *(const bf16x8 *)(Vs + lds_off<8>(vrow, 4 + hi)), p1a, acc[nb], 0, 0, 0);
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        *(const bf16x8 *)(Vs + lds_off<8>(vrow, 6 + hi)), p1b, acc[nb], 0, 0, 0);
                }
            }
        }

        if (more)
            store_stage<D>(stK, stV, smem + (buf ^ 1) * STAGE_BYTES, tid);
        buf ^= 1;
        idx = nidx;
        half = nhalf;
    }

    if (wave_active) {
        const float lt = l_run + __shfl_xor(l_run, 32);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        uint16_t *orow = Op + qrow * D;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                // O^T accumulator register 4 g + u of lane l holds feature
                // 32 nb + 8 g + 4 hi + u of query l32.
                union {
                    __bf16 b[4];
                    uint2 u;
                } pk;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    pk.b[u] = (__bf16)(acc[nb][4 * g + u] * inv);
                *(uint2 *)(orow + 32 * nb + 8 * g + 4 * hi) = pk.u;
            }
        }
    }
}

}  // namespace

hipError_t launch_attention_mfma(const Layout &L, const AttnParams &p, hipStream_t s)
{
    const dim3 grid(L.heads * L.nT);
    if (L.D == 128)
        hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, dim3(kThreads), 0, s, L, p);
    else
        hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, dim3(kThreads), 0, s, L, p);
    return hipGetLastError();
}

}  // namespace sa
