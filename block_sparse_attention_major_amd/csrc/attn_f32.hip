// Block-sparse flash attention forward in fp32 on the gfx950 matrix cores
// (v_mfma_f32_32x32x2_f32): fp32 Q, K, V, scores, probabilities and
// accumulation, one query tile per workgroup.
//
// What is computed: for every query tile i of head h, exact softmax
// attention over the keys of the key tiles its mask row keeps (Compact
// Attention page, Fig. 3 caption: precomputed masks run in block-sparse
// attention kernels; SCOPE review page, abstract: attention over the selected
// original keys and values).  Dropped tile pairs cost no loads and no FLOPs.
//
// Design (ours, for CDNA4; the pages give no kernel design):
//  - One workgroup of 4 waves per (head, query tile), 32 query slots per
//    wave; two workgroups share a CU.  The tile-major layout of the fp32
//    path is used as it is (tile tau at rows tau S, S = tile volume): no
//    transposed V and no 128-slot padding.
//  - Keys are consumed in stages of 32.  The K rows and the V rows of a
//    stage are copied global -> LDS by the DMA path (buffer_load_dwordx4 ...
//    lds) into one of two buffers, one stage ahead of the math; rows past
//    the stage's real keys are read but masked (past the end of the head's
//    buffer the loads return zero).
//  - Scores are computed transposed, S^T = K Q^T: one product takes two
//    features, the lane's half l / 32 picking which, so the lanes of half 0
//    walk features 0 .. D/2 - 1 and those of half 1 features D/2 .. D - 1,
//    and a lane holds its D/2 features of its query in registers; K operands
//    are 16-byte LDS reads of four k-steps.  Result register v of lane l is
//    key 8 (v / 4) + 4 (l / 32) + v % 4 of query l % 32, which is also the
//    B-operand order of O^T += V^T P^T (k-step v: key 8 (v / 4) + v % 4 for
//    half 0, 4 more for half 1), so the probabilities feed the second
//    product from their own registers.
//  - The fp32 matrix rate is low enough (a 32 x 32 x 2 product every 64
//    clocks) that the matrix cores, not the softmax, bound the step: the
//    softmax is the classic one (row maximum per stage, rescale) in fp32.
//  - LDS rows are XOR-swizzled in 16-byte chunks: K by the row (the 32 rows
//    of one operand read land on distinct chunks), V by bit 2 of the row
//    (the two lane halves read rows 4 apart).
#include "mfma_util.h"

namespace sa {

namespace {

using namespace mfma;

constexpr int kThreads = 256;  // 4 waves
constexpr int kKeys = 32;      // keys per stage
constexpr int kList = 2048;    // key-tile ids staged in LDS at a time

__device__ __forceinline__ int tile_tokens(const Layout &L, const AttnParams &P, int j)
{
    return mfma::tile_tokens(L, P.div_plane, P.div_row, j);
}

template <int D>
struct F32Stage {
    static constexpr int ROWB = D * 4;           // bytes of a K or V row
    static constexpr int RC = D / 4;             // 16-byte chunks per row
    static constexpr int PART = kKeys * ROWB;    // bytes of the stage's K (or V)
    static constexpr int BLK = PART / 1024;      // 1 KB DMA blocks per part
    static constexpr int BPW = 2 * BLK / 4;      // blocks per wave
    static_assert(BLK % BPW == 0, "a wave moves K blocks or V blocks, not both");
};

// XOR terms of the LDS chunk positions.
template <int D>
__device__ __forceinline__ int k_swz(int row)
{
    return row & (F32Stage<D>::RC - 1);
}
__device__ __forceinline__ int v_swz(int row) { return ((row >> 2) & 1) * 8; }

template <int D>
struct F32Dma {
    __amdgpu_buffer_rsrc_t rsrc;      // K or V rows of head h
    bool is_v;                        // wave-uniform
    int off[F32Stage<D>::BPW];        // byte offset of the lane's chunk within a stage
};

// LDS byte 16 l of a DMA block receives lane l's 16 bytes, so each lane
// fetches the global chunk that the swizzle puts there.
template <int D>
__device__ __forceinline__ void make_dma(F32Dma<D> &pl, const float *Kp, const float *Vp, const Layout &L,
                                         int h, int wave, int lane)
{
    constexpr int BLK = F32Stage<D>::BLK, BPW = F32Stage<D>::BPW, ROWB = F32Stage<D>::ROWB;
    pl.is_v = wave * BPW >= BLK;
    const float *base = (pl.is_v ? Vp : Kp) + (long long)h * L.Npad * D;
    // Raw buffer over one head's rows (N_pad D 4 bytes < 2^31, checked when
    // the handle is created); loads past it return zero.
    pl.rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)(L.Npad * D * 4), 0x00020000);
#pragma unroll
    for (int t = 0; t < BPW; ++t) {
        const int blk = wave * BPW + t - (pl.is_v ? BLK : 0);
        const int pos = blk * 1024 + 16 * lane;
        const int row = pos / ROWB, ph = (pos % ROWB) >> 4;
        const int c = ph ^ (pl.is_v ? v_swz(row) : k_swz<D>(row));
        pl.off[t] = row * ROWB + 16 * c;
    }
}

// Copies stage `st` (keys 32 st ..) of key tile j into the stage buffer.
template <int D>
__device__ __forceinline__ void issue_stage(const F32Dma<D> &pl, lds_char *stage, int j, int st, int S, int wave)
{
    constexpr int BPW = F32Stage<D>::BPW;
    const int soff = (j * S + st * kKeys) * D * 4;
    lds_char *dst = stage + wave * BPW * 1024;
#pragma unroll
    for (int t = 0; t < BPW; ++t)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pl.rsrc, (__attribute__((address_space(3))) void *)(dst + t * 1024),
                                                 16, pl.off[t], soff, 0, 0);
}

template <int D>
struct F32State {
    f32x16 acc[D / 32];  // O^T: register v of block nb = feature 32 nb + 8 (v / 4) + 4 (l / 32) + v % 4
    float m, l;          // running max (log2 units) and this lane's partial row sum
};

// One stage: S^T = K Q^T over its kv real keys, online softmax, O^T += V^T P^T.
// Ks: K rows, Vs: V rows of the stage; kb: the lane's K base offset, vb[nb]
// its V base offsets.
template <int D>
__device__ __forceinline__ void attend_stage(const char *Ks, const char *Vs, const float (&qf)[D / 2], int kb,
                                             const int (&vb)[D / 32], int kv, float sl2, int hi, F32State<D> &st)
{
    constexpr int NB = D / 32, ROWB = F32Stage<D>::ROWB;
    // Two accumulators (even and odd groups of four k-steps) halve the chain
    // of dependent products.
    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int g = 0; g < D / 8; ++g) {
        const float4 a = *(const float4 *)(Ks + (kb ^ (g << 4)));
        f32x16 &s = (g & 1) ? s1 : s0;
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, qf[4 * g], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, qf[4 * g + 1], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, qf[4 * g + 2], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, qf[4 * g + 3], s, 0, 0, 0);
    }
    float p[16];
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int key = 8 * (v >> 2) + 4 * hi + (v & 3);
        p[v] = key < kv ? s0[v] + s1[v] : -INFINITY;
        mx = fmaxf(mx, p[v]);
    }
    // Key 0 is real (kv >= 1), so the row maximum is finite.
    const float m_new = fmaxf(st.m, half_max(mx) * sl2);
    const float alpha = exp2_fast(st.m - m_new);
    float ls = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        p[v] = exp2_fast(fmaf(p[v], sl2, -m_new));
        ls += p[v];
    }
    st.m = m_new;
    st.l = fmaf(st.l, alpha, ls);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
            st.acc[nb][v] *= alpha;
    }
    // k-step v takes key 8 (v / 4) + v % 4 (half 0) or that + 4 (half 1):
    // V row offset (8 (v / 4) + v % 4) ROWB from the lane's base.
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int roff = (8 * (v >> 2) + (v & 3)) * ROWB;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float a = *(const float *)(Vs + vb[nb] + roff);
            st.acc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[v], st.acc[nb], 0, 0, 0);
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_f32_kernel(Layout L, AttnParams P)
{
    constexpr int NB = D / 32, PART = F32Stage<D>::PART, ROWB = F32Stage<D>::ROWB, RC = F32Stage<D>::RC;
    __shared__ __attribute__((aligned(1024))) char buf0[2 * PART];
    __shared__ __attribute__((aligned(1024))) char buf1[2 * PART];
    __shared__ int clist[kList];

    const float *__restrict__ Qp = (const float *)P.q;
    const float *__restrict__ Kp = (const float *)P.k;
    const float *__restrict__ Vp = (const float *)P.v;
    float *__restrict__ Op = (float *)P.o;
    const int *__restrict__ cols = P.rows.cols;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const int ci = tile_tokens(L, P, i);
    const bool wave_active = wave * 32 < ci;

    // This lane's query: slot 32 wave + l % 32 of tile i.
    const int slot = wave * 32 + l32;
    const bool q_real = slot < ci;
    const int tok = (q_real && (P.raster || P.lse)) ? raster_token(L, i, slot) : 0;
    const long long qrow = P.raster ? (long long)h * L.N + tok : (long long)h * L.Npad + (long long)i * L.S + slot;
    const bool q_io = wave_active && q_real;
    float *lse_at = (P.lse && q_real && hi == 0) ? P.lse + (long long)h * L.N + tok : nullptr;

    // Q operand (B of S^T = K Q^T): features hi D/2 .. hi D/2 + D/2 - 1 of the
    // lane's query.
    float qf[D / 2];
    if (q_io) {
        const float4 *qp = (const float4 *)(Qp + qrow * D + hi * (D / 2));
#pragma unroll
        for (int g = 0; g < D / 8; ++g) {
            const float4 x = qp[g];
            qf[4 * g] = x.x;
            qf[4 * g + 1] = x.y;
            qf[4 * g + 2] = x.z;
            qf[4 * g + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int u = 0; u < D / 2; ++u)
            qf[u] = 0.f;
    }
    F32State<D> st;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            st.acc[nb][v] = 0.f;
    st.m = -INFINITY;
    st.l = 0.f;
    const float sl2 = P.scale_log2;

    // Per-lane LDS offsets.  K: row l % 32, chunk hi RC/2 + g at
    // kb ^ (g << 4).  V: row 4 hi (+ the k-step's row), chunk 8 nb + (l % 32)
    // / 4 swizzled by 8 hi, word l % 4: (vb0 ^ 128 nb).
    const int kb = l32 * ROWB + (((hi * (RC / 2)) ^ k_swz<D>(l32)) << 4);
    int vb[NB];
    {
        const int vb0 = 4 * hi * ROWB + ((((l32 >> 2) ^ (8 * hi)) << 4) + 4 * (l32 & 3));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            vb[nb] = vb0 ^ (128 * nb);
    }

    const int beg = P.rows.row_ptr[r];
    const int end = (int)min((long long)P.rows.row_ptr[r + 1], P.rows.cap);
    int list_base = beg, list_end = beg;
    auto fill_list = [&](int from) {
        list_base = from;
        list_end = min(end, from + kList);
        for (int u = tid; u < list_end - list_base; u += kThreads)
            clist[u] = cols[list_base + u];
        __syncthreads();
    };

    F32Dma<D> dma;
    make_dma<D>(dma, Kp, Vp, L, h, wave, lane);

    // Stage cursor: key tile idx (id j, c real tokens) and its 32-key stage.
    int idx = beg, sg = 0, j = 0, c = 0;
    if (idx < end) {
        fill_list(beg);
        j = __builtin_amdgcn_readfirstlane(clist[0]);
        c = tile_tokens(L, P, j);
        issue_stage<D>(dma, (lds_char *)buf0, j, 0, L.S, wave);
    }
    auto advance = [&]() {
        if ((sg + 1) * kKeys < c) {
            ++sg;
        } else {
            ++idx;
            sg = 0;
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
        {
            const int kv = min(kKeys, c - sg * kKeys);
            wait_vmcnt<0>();
            __syncthreads();  // buf0 complete; buf1 free
            advance();
            if (idx < end)
                issue_stage<D>(dma, (lds_char *)buf1, j, sg, L.S, wave);
            if (wave_active)
                attend_stage<D>(buf0, buf0 + PART, qf, kb, vb, kv, sl2, hi, st);
        }
        if (idx >= end)
            break;
        {
            const int kv = min(kKeys, c - sg * kKeys);
            wait_vmcnt<0>();
            __syncthreads();  // buf1 complete; buf0 free
            advance();
            if (idx < end)
                issue_stage<D>(dma, (lds_char *)buf0, j, sg, L.S, wave);
            if (wave_active)
                attend_stage<D>(buf1, buf1 + PART, qf, kb, vb, kv, sl2, hi, st);
        }
    }
    wait_vmcnt<0>();  // no copy may land after the workgroup ends

    if (!wave_active)
        return;
    const float lt = half_sum(st.l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (lse_at)
        *lse_at = lt > 0.f ? (st.m + log2f(lt)) * kLn2 : -INFINITY;
    if (q_io) {
        float *orow = Op + qrow * D;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 x = {st.acc[nb][4 * g] * inv, st.acc[nb][4 * g + 1] * inv, st.acc[nb][4 * g + 2] * inv,
                                  st.acc[nb][4 * g + 3] * inv};
                *(float4 *)(orow + 32 * nb + 8 * g + 4 * hi) = x;
            }
        }
    }
}

}  // namespace

hipError_t launch_attention_f32(const Layout &L, const AttnParams &p, hipStream_t s)
{
    const dim3 grid(L.heads * L.nT);
    if (L.D == 128)
        hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(kThreads), 0, s, L, p);
    else
        hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(kThreads), 0, s, L, p);
    return hipGetLastError();
}

}  // namespace sa
