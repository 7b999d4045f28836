// Block-sparse flash attention forward over single query tiles (the row
// kernel), bf16 in / fp32 accumulate, on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16).  It serves the query tiles whose pair the
// mask compiler did not give to the pair kernel (attn_mfma.hip): pairs whose
// two key lists overlap too little for a shared key stream to pay off, and
// tiles left alone at an odd edge of the tile grid.
//
// What is computed: for every query tile i of head h, exact softmax
// attention over the keys of the key tiles its mask row keeps (Compact
// Attention page, Fig. 3 caption: precomputed masks run in block-sparse
// attention kernels; SCOPE review page, abstract: attention over the selected
// original keys and values).  Dropped tile pairs cost no loads and no FLOPs.
//
// Design (ours, for CDNA4; the pages give no kernel design):
//  - One workgroup of 4 waves per (head, query tile); tile = 128 slots, each
//    wave owns 32 query slots.  Two workgroups share a CU, so each SIMD runs
//    two independent waves and overlaps one's softmax with the other's MFMAs;
//    a wave raises its issue priority for its softmax, which bounds the step.
//    Workgroups follow the compiled longest-first order, remapped so each XCD
//    (which owns its L2) takes contiguous chunks of it: neighbouring rows
//    share key tiles.
//  - Keys are consumed in stages of 64 (half a tile).  K and the transposed V
//    tile of a stage are copied global -> LDS by the DMA path
//    (buffer_load_dwordx4 ... lds: no registers, no LDS store instructions;
//    the buffer form keeps the compiler's LDS waits precise while copies are
//    in flight) into one of two statically addressed buffers, one stage
//    ahead of the math.
//    The empty tail of a clipped key tile (80 of 128 slots at 720p) is
//    skipped at 32-key granularity.
//  - Scores are computed transposed, S^T = K Q^T, so each lane holds 16 keys
//    of one query: row max and row sum are in-lane, plus one exchange with
//    the lane 32 apart (v_permlane32_swap).  K rows are fed to the MFMA in a
//    permuted order so the probabilities come out already in the operand
//    order of the next product, O^T += V^T P^T, whose accumulator again keeps
//    one query per lane (the rescale is in-lane).
//  - V arrives pre-transposed per tile ([D][128], written by the permute
//    stage), so V^T operand reads are plain 16-byte LDS reads.
//  - LDS rows are XOR-swizzled in 16-byte chunks so the MFMA operand reads hit
//    16 distinct chunk positions per 16 lanes.
//  - Online softmax in fp32 and exp2 against a running reference that is
//    moved only on a rare wave-uniform redo (no row maximum per stage; see
//    online_softmax in mfma_util.h); row sums are taken from the bf16
//    probabilities with v_dot2.
//  - Q and O rows go to the caller's raster tensors or the tile-major
//    workspace, and the log-sum-exp is written on request, as in the pair
//    kernel.
#include "mfma_util.h"

namespace sa {

namespace {

using namespace mfma;

constexpr int kThreads = 256;
constexpr int kList = 2048;  // key-tile ids staged in LDS at a time

// Real tokens of tile j.
__device__ __forceinline__ int tile_tokens(const Layout &L, const AttnParams &P, int j)
{
    return mfma::tile_tokens(L, P.div_plane, P.div_row, j);
}

// One stage (64 keys, half `half` of key tile j) in LDS: K rows [64][D] then
// transposed V [D][64], both swizzled.  The stage is 2 * D KB, moved as 1 KB
// DMA blocks of 64 lanes x 16 bytes; LDS byte 16 l of a block receives lane
// l's load, so each lane fetches the global chunk that the swizzle puts
// there.  Wave w moves blocks [w * BPW, (w + 1) * BPW): the first half of the
// waves moves K, the second half V^T.
template <int D>
struct RowDma {
    static constexpr int KBLK = kStage * D * 2 / 1024;  // K blocks per stage (V^T has as many)
    static constexpr int BPW = 2 * KBLK / 4;            // blocks per wave
    static_assert(KBLK % BPW == 0, "a wave moves K blocks or V^T blocks, not both");
    __amdgpu_buffer_rsrc_t rsrc;  // K of head h, or V^T of head h (N_pad D 2 bytes)
    bool is_v;                    // wave-uniform
    int off[BPW];                 // byte offset of the lane's chunk within a stage
};

template <int D>
__device__ __forceinline__ void make_row_dma(RowDma<D> &pl, const uint16_t *Kp, const uint16_t *Vt,
                                             const Layout &L, int h, int wave, int lane)
{
    constexpr int KBLK = RowDma<D>::KBLK, BPW = RowDma<D>::BPW;
    pl.is_v = wave * BPW >= KBLK;
    const char *base = pl.is_v ? (const char *)(Vt + (long long)h * L.nT * D * kTile)
                               : (const char *)(Kp + (long long)h * L.Npad * D);
    // Raw buffer over one head's K (or V^T): N_pad D 2 bytes, below 2^31
    // because the plan keeps heads * tiles^2 below 2^31, so the stage's
    // byte offset (scalar) and the lane's offset in it (vector) both fit 32
    // bits.  Word 3 is the gfx9 raw 32-bit data format.
    pl.rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, L.Npad * D * 2, 0x00020000);
#pragma unroll
    for (int t = 0; t < BPW; ++t) {
        const int blk = wave * BPW + t;
        pl.off[t] = pl.is_v ? vt_chunk_src(blk - KBLK, lane) : k_chunk_src<D>(blk, lane);
    }
}

// Issue this wave's DMA blocks of stage (key tile j, half `half`) into the
// stage buffer at `stage`.  j and wave are wave-uniform (read with
// readfirstlane), so the stage offset and the LDS destinations are scalars
// and the eight copies issue without branches.
template <int D>
__device__ __forceinline__ void issue_stage(const RowDma<D> &pl, lds_char *stage, int j, int half, int wave)
{
    constexpr int BPW = RowDma<D>::BPW;
    const int soff = pl.is_v ? (j * D * kTile + half * kStage) * 2 : (j * kTile + half * kStage) * D * 2;
    lds_char *dst = stage + wave * BPW * 1024;
#pragma unroll
    for (int t = 0; t < BPW; ++t)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pl.rsrc, (__attribute__((address_space(3))) void *)(dst + t * 1024),
                                                 16, pl.off[t], soff, 0, 0);
}

// Attention of this wave's 32 queries to the kv real keys (1..64) of the
// stage held in LDS at Ks (K) and Ks + K_BYTES (V^T).
template <int D>
__device__ __forceinline__ void attend_stage(const char *Ks, const bf16x8 (&qf)[D / 16], int kv,
                                             float sl2, int prow, int l32, int hi, RowState<D> &st)
{
    constexpr int KS = D / 16, NB = D / 32, RCK = D / 8;
    constexpr int K_BYTES = kStage * D * 2;
    const char *Vs = Ks + K_BYTES;
    const bool two = kv > 32;
    Scores S;
    f32x16 &s0 = S.s0, &s1 = S.s1;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
        s0[jj] = 0.f;
        s1[jj] = 0.f;
    }
    if (two) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a0 = *(const bf16x8 *)(Ks + lds_off<RCK>(prow, 2 * ks + hi));
            const bf16x8 a1 = *(const bf16x8 *)(Ks + lds_off<RCK>(32 + prow, 2 * ks + hi));
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], s1, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                *(const bf16x8 *)(Ks + lds_off<RCK>(prow, 2 * ks + hi)), qf[ks], s0, 0, 0, 0);
    }
    // From here to the P V products the wave runs its softmax at raised
    // issue priority: the other workgroup's wave on this SIMD is then most
    // often in its matrix products, and the exponentials, which bound the
    // step, get the issue slots first.
    __builtin_amdgcn_s_setprio(2);
    if (kv < kStage)
        mask_stage_tail(S, kv, hi);
    Probs Pr;
    online_softmax<D>(Pr, S, kv, sl2, st);
    const bf16x8 &p0a = Pr.p[0], &p0b = Pr.p[1], &p1a = Pr.p[2], &p1b = Pr.p[3];
    // O^T += V^T P^T: A operand = V^T rows 32 nb + l32, keys in 16-key steps.
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        st.acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *(const bf16x8 *)(Vs + lds_off<8>(32 * nb + l32, 0 + hi)), p0a, st.acc[nb], 0, 0, 0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        st.acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *(const bf16x8 *)(Vs + lds_off<8>(32 * nb + l32, 2 + hi)), p0b, st.acc[nb], 0, 0, 0);
    if (two) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            st.acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                *(const bf16x8 *)(Vs + lds_off<8>(32 * nb + l32, 4 + hi)), p1a, st.acc[nb], 0, 0, 0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            st.acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                *(const bf16x8 *)(Vs + lds_off<8>(32 * nb + l32, 6 + hi)), p1b, st.acc[nb], 0, 0, 0);
    }
}

// Wait for this wave's outstanding vector-memory operations (the stage DMA),
// leaving LDS and scalar counters alone.
__device__ __forceinline__ void wait_vmem() { wait_vmcnt<0>(); }

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_rows_kernel(Layout L, AttnParams P)
{
    constexpr int KS = D / 16;
    constexpr int NB = D / 32;
    constexpr int STAGE_BYTES = 2 * kStage * D * 2;
    __shared__ __attribute__((aligned(1024))) char buf0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char buf1[STAGE_BYTES];
    __shared__ int clist[kList];

    const uint16_t *__restrict__ Qp = (const uint16_t *)P.q;
    const uint16_t *__restrict__ Kp = (const uint16_t *)P.k;
    const uint16_t *__restrict__ Vt = (const uint16_t *)P.v;
    uint16_t *__restrict__ Op = (uint16_t *)P.o;
    const int *__restrict__ cols = P.rows.cols;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep it scalar
    const int l32 = lane & 31, hi = lane >> 5;

    // XCD-aware remap: workgroup b runs on XCD b % 8; give each XCD
    // contiguous chunks of the work order.
    int w = blockIdx.x;
    {
        const int C = P.xcd_chunk;
        const int G = gridDim.x;
        const int G8 = C > 0 ? (G / (8 * C)) * (8 * C) : 0;
        if (w < G8) {
            const int xcd = w & 7, slot = w >> 3;
            w = ((slot / C) * 8 + xcd) * C + slot % C;
        }
    }
    const int r = P.rows.order[w];
    const int h = r / L.nT, i = r - h * L.nT;
    if (P.pair_flag[h * L.nP + tile_pair(L, i)])
        return;  // the pair kernel serves this tile
    const int ci = tile_tokens(L, P, i);
    const bool wave_active = wave * 32 < ci;

    // This lane's query: slot wave * 32 + l32 of tile i, a real token when
    // the slot is below c_i.  Its row in q and o is the raster token
    // (raster I/O, real slots only) or the tile-major slot.
    const int slot = wave * 32 + l32;
    const bool q_real = slot < ci;
    const int tok = (q_real && (P.raster || P.lse)) ? raster_token(L, i, slot) : 0;
    const long long qrow = P.raster ? (long long)h * L.N + tok
                                    : (long long)h * L.Npad + (long long)i * kTile + slot;
    const bool q_io = q_real || !P.raster;
    // Where this query's log-sum-exp goes (one lane per query), or null.
    float *lse_at = (P.lse && q_real && hi == 0) ? P.lse + (long long)h * L.N + tok : nullptr;

    // Q operand (B of S^T = K Q^T): lane holds query l32, features
    // 16 ks + 8 hi .. +7 for every k-step.
    bf16x8 qf[KS];
    if (q_io) {
        const bf16x8 *qp = (const bf16x8 *)(Qp + qrow * D);
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
    RowState<D> st;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            st.acc[nb][jj] = 0.f;
    st.m = -INFINITY;
    st.l = 0.f;
    const float sl2 = P.scale_log2;

    const int beg = P.rows.row_ptr[r];
    const int end = (int)min((long long)P.rows.row_ptr[r + 1], P.rows.cap);

    // The row's key-tile ids, staged in LDS (kList at a time; longer rows
    // refill the list when the cursor reaches its end).
    int list_base = beg, list_end = beg;
    auto fill_list = [&](int from) {
        list_base = from;
        list_end = min(end, from + kList);
        for (int u = tid; u < list_end - list_base; u += kThreads)
            clist[u] = cols[list_base + u];
        __syncthreads();
    };

    RowDma<D> dma;
    make_row_dma<D>(dma, Kp, Vt, L, h, wave, lane);

    // Stage cursor: key tile idx (id j, c real tokens) and which half of it.
    int idx = beg, half = 0, j = 0, c = 0;
    if (idx < end) {
        fill_list(beg);
        j = __builtin_amdgcn_readfirstlane(clist[0]);
        c = tile_tokens(L, P, j);
        issue_stage<D>(dma, (lds_char *)buf0, j, 0, wave);
    }
    const int prow = key_of_mfma_row(l32);

    // Advance the cursor by one stage (all waves together, after a barrier).
    auto advance = [&]() {
        if (half == 0 && c > kStage) {
            half = 1;
        } else {
            ++idx;
            half = 0;
            if (idx < end) {
                if (idx == list_end) {
                    __syncthreads();  // every wave is done reading the list
                    fill_list(idx);
                }
                j = __builtin_amdgcn_readfirstlane(clist[idx - list_base]);
                c = tile_tokens(L, P, j);
            }
        }
    };

    while (idx < end) {
        // ---- stage in buf0
        {
            const int kv = min(kStage, c - half * kStage);
            wait_vmem();
            __syncthreads();  // buf0 complete; buf1 free
            advance();
            if (idx < end)
                issue_stage<D>(dma, (lds_char *)buf1, j, half, wave);
            if (wave_active)
                attend_stage<D>(buf0, qf, kv, sl2, prow, l32, hi, st);
        }
        if (idx >= end)
            break;
        // ---- stage in buf1
        {
            const int kv = min(kStage, c - half * kStage);
            wait_vmem();
            __syncthreads();  // buf1 complete; buf0 free
            advance();
            if (idx < end)
                issue_stage<D>(dma, (lds_char *)buf0, j, half, wave);
            if (wave_active)
                attend_stage<D>(buf1, qf, kv, sl2, prow, l32, hi, st);
        }
    }

    if (wave_active)
        finish_rows<D>(st, true, lse_at, q_io ? Op + qrow * D : nullptr, hi);
}

}  // namespace

hipError_t launch_attention_rows(const Layout &L, const AttnParams &p, hipStream_t s)
{
    const dim3 grid(L.heads * L.nT);
    if (L.D == 128)
        hipLaunchKernelGGL(attn_rows_kernel<128>, grid, dim3(kThreads), 0, s, L, p);
    else
        hipLaunchKernelGGL(attn_rows_kernel<64>, grid, dim3(kThreads), 0, s, L, p);
    return hipGetLastError();
}

}  // namespace sa
