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
// (waves 0-3 tile 2r, waves 4-7 tile 2r + 1, 32 queries per wave).  Key
// tiles stream through two LDS buffers: while the waves work on tile j, the
// DMA path (buffer_load_dwordx4 ... lds, one 1 KB block per instruction,
// each wave its share) brings tile j + 1 into the other buffer.  Rows are
// XOR-swizzled in 16-byte chunks, so the operand reads of 16 consecutive
// rows at one column hit 16 distinct chunk positions.  Each wave reads the
// staged tile as the A operand of v_mfma_f32_32x32x16_bf16 (S^T = K Q^T; Q
// stays in registers as the B operand); lane l then holds the scores of
// query l % 32 against 16 keys of each 32-key block.  Per key tile, each
// wave's pass-2 partial sum goes to LDS and one thread per query tile adds
// the four after the next barrier.  Two workgroups share a CU; a wave raises
// its issue priority for the exponentials of each block.
#include "mfma_util.h"

namespace sa {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileRows = 128;

using namespace mfma;

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
    constexpr int RC = D / 8;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        acc[r] = 0.f;
    const int row = kb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = *(const bf16x8 *)(Ks + lds_off<RC>(row, 2 * ks + hi));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], acc, 0, 0, 0);
    }
    return acc;
}

// Keys past cj (the tile's real count) score -inf.
__device__ __forceinline__ void mask_tail(f32x16 &s, int kb, int cj, int hi)
{
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r / 4) + 4 * hi + r % 4;
        if (key >= cj)
            s[r] = -INFINITY;
    }
}

// One 1 KB DMA block: lane l's 16 bytes at byte voff + soff of the buffer
// land at LDS byte 16 l of dst.
__device__ __forceinline__ void dma_block(__amdgpu_buffer_rsrc_t rs, char *dst, int voff, int soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)dst, 16, voff, soff,
                                             0, 0);
}

// s_waitcnt on this wave's vector-memory counter only (vmcnt(0)).
__device__ __forceinline__ void wait_vm0() { wait_vmcnt<0>(); }

template <int D>
__global__ __launch_bounds__(kThreads, 1) void mass_kernel(Layout L, const uint16_t *__restrict__ Qt,
                                                           const uint16_t *__restrict__ Kt,
                                                           float scale_log2, float *__restrict__ mass)
{
    constexpr int KS = D / 16;
    constexpr int TILE = kTileRows * D * 2;             // bytes of a staged key tile
    constexpr int BLK = TILE / 1024;                    // 1 KB DMA blocks per tile
    constexpr int BPW = BLK / kWaves;                   // blocks per wave
    static_assert(BPW * kWaves == BLK, "DMA blocks spread evenly over the waves");
    __shared__ __attribute__((aligned(1024))) char Kb0[TILE];
    __shared__ __attribute__((aligned(1024))) char Kb1[TILE];
    __shared__ float part[2][kWaves];

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
            (const bf16x8 *)(Qt + ((long long)h * L.Npad + (long long)i * L.S + slot) * D);
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

    // DMA of key tile j into a buffer: raw buffer over the head's permuted K
    // (N_pad D 2 bytes < 2^31); LDS byte 16 l of a block receives lane l's
    // 16 bytes, so each lane fetches the chunk the swizzle puts there.
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(Kt + (long long)h * L.Npad * D), 0, L.Npad * D * 2, 0x00020000);
    int voff[BPW];
#pragma unroll
    for (int t = 0; t < BPW; ++t)
        voff[t] = k_chunk_src<D>(wave * BPW + t, lane);
    auto stage = [&](char *buf, int j) {
        const int soff = j * TILE;
#pragma unroll
        for (int t = 0; t < BPW; ++t)
            dma_block(krs, buf + (wave * BPW + t) * 1024, voff[t], soff);
    };

    // One pass over every key tile: before tile j is used, every wave waits
    // for its own copies of j and the barrier for everyone's; then tile j + 1
    // goes to the other buffer, which every wave left in the previous step.
    // visit(j, Ks) does the work of tile j.
    float m = -INFINITY, l = 0.f, lse2 = 0.f;
    auto visit1 = [&](int j, const char *Ks) {
        const int cj = tile_real_count(L, j);
        if (!wave_active)
            return;
        for (int kb = 0; kb * 32 < cj; ++kb) {
            f32x16 s = block_scores<D>(Ks, kb, qf, l32, hi);
            if (kb * 32 + 32 > cj)
                mask_tail(s, kb, cj, hi);
            // The exponentials of a block run at raised issue priority: the
            // other workgroup's waves on this SIMD are then most often in
            // their matrix products, and the exponentials bound the loop.
            __builtin_amdgcn_s_setprio(2);
            float mx = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r)
                mx = fmaxf(mx, s[r]);
            const float m_new = fmaxf(m, mx * scale_log2);
            if (m_new > -INFINITY) {
                l *= __builtin_amdgcn_exp2f(m - m_new);
                m = m_new;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    l += __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -m));
            }
            __builtin_amdgcn_s_setprio(0);
        }
    };
    // Pass 2: the partial sums of tile j go to part[j & 1] and are added up
    // after the next barrier.
    auto flush = [&](int j) {
        if (tid < 2 && i0 + tid < L.nT) {
            const int t = i0 + tid;
            const float *pp = part[j & 1] + 4 * tid;
            mass[((long long)h * L.nT + t) * L.nT + j] = (pp[0] + pp[1] + pp[2] + pp[3]) / (float)tile_real_count(L, t);
        }
    };
    auto visit2 = [&](int j, const char *Ks) {
        if (j > 0)
            flush(j - 1);
        const int cj = tile_real_count(L, j);
        float acc = 0.f;
        if (wave_active) {
            for (int kb = 0; kb * 32 < cj; ++kb) {
                f32x16 s = block_scores<D>(Ks, kb, qf, l32, hi);
                if (kb * 32 + 32 > cj)
                    mask_tail(s, kb, cj, hi);
                __builtin_amdgcn_s_setprio(2);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc += __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -lse2));
                __builtin_amdgcn_s_setprio(0);
            }
        }
        acc = wave_sum(q_real ? acc : 0.f);
        if (lane == 0)
            part[j & 1][wave] = acc;
    };
    auto visit = [&](int which, int j, const char *Ks) {
        if (which == 0)
            visit1(j, Ks);
        else
            visit2(j, Ks);
    };
    auto pass = [&](int which) {
        stage(Kb0, 0);
#pragma unroll 1
        for (int j = 0; j < L.nT; j += 2) {
            wait_vm0();
            lds_barrier();
            if (j + 1 < L.nT)
                stage(Kb1, j + 1);
            visit(which, j, (const char *)Kb0);
            if (j + 1 < L.nT) {
                wait_vm0();
                lds_barrier();
                if (j + 2 < L.nT)
                    stage(Kb0, j + 2);
                visit(which, j + 1, (const char *)Kb1);
            }
        }
    };

    // Pass 1: running max (log2 units) and sum over every key.
    pass(0);
    // Lanes l and l ^ 32 hold different keys of the same query.
    const float m_o = __shfl_xor(m, 32), l_o = __shfl_xor(l, 32);
    const float m_all = fmaxf(m, m_o);
    const float l_all = (m > -INFINITY ? l * exp2f(m - m_all) : 0.f) +
                        (m_o > -INFINITY ? l_o * exp2f(m_o - m_all) : 0.f);
    lse2 = m_all + log2f(l_all);
    // Pass 2: mass per key tile.
    lds_barrier();  // every wave is done with pass 1's buffers
    pass(1);
    lds_barrier();
    flush(L.nT - 1);
    wait_vm0();
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
