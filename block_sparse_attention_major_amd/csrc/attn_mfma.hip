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
//  - One workgroup of 8 waves per pair of query tiles of one head (tiles
//    next to each other along y, t or x; see pair_tiles), one workgroup per
//    CU.  Waves 0-3 (group A) serve the first tile, waves 4-7 (group B) the
//    second, 32 query slots per wave.  Both walk the union of the two key
//    lists, so a key tile kept by both is loaded once for 256 queries; each
//    list entry says which of the two keeps it, and a group skips the math
//    of entries its tile does not keep.
//  - Ping-pong: each SIMD hosts one wave of each group; A's step runs its
//    matrix products and then its softmax, B's step the softmax of the
//    previous stage and then its products, so while one of the two issues
//    matrix products the other runs its exponentials, with one workgroup
//    barrier per step (schedule in the kernel body).
//  - Keys are consumed in stages of 64 (half a key tile).  K and the
//    transposed V tile of a stage are copied global -> LDS by the DMA path
//    (buffer_load_dwordx4 ... lds: no registers, no LDS store instructions)
//    into a ring of four statically addressed slots, two stages ahead of
//    the math, issued at the start of the softmax phase (the other group's
//    wave keeps the matrix core busy meanwhile).  The buffer form, unlike
//    the global one, lets the compiler count the LDS operand reads
//    precisely while copies are in flight (with a global-to-LDS copy
//    pending it waits for every outstanding LDS read at each use, which
//    defeats the read-ahead).  The empty tail
//    of a clipped key tile (80 of 128 slots at 720p) is skipped at 32-key
//    granularity.
//  - Workgroups follow the compiled longest-first order of the pair lists,
//    remapped so each XCD (which owns its L2) takes contiguous chunks of it:
//    neighbouring pairs share key tiles.
//  - Scores are computed transposed, S^T = K Q^T, so each lane holds 16 keys
//    of one query: row max and row sum are in-lane, plus one exchange with
//    the lane 32 apart (v_permlane32_swap).  K rows are fed to the MFMA in a
//    permuted order so the probabilities come out already in the operand
//    order of the next product, O^T += V^T P^T, whose accumulator again keeps
//    one query per lane (the rescale is in-lane).
//  - V arrives pre-transposed per tile ([D][128], written by the permute
//    stage), so V^T operand reads are plain 16-byte LDS reads, issued one
//    key step ahead of the products that use them (K operand reads two
//    k-steps ahead).
//  - LDS rows are XOR-swizzled in 16-byte chunks so the MFMA operand reads hit
//    16 distinct chunk positions per 16 lanes.
//  - Online softmax in fp32 and exp2 against a running reference that is
//    moved only on a rare wave-uniform redo (no row maximum per stage; see
//    online_softmax in mfma_util.h); row sums are taken from the bf16
//    probabilities with v_dot2.
//  - Each lane reads its query row of Q and writes its row of O either in
//    the caller's raster tensors (the forward: the Q permute and O
//    unpermute are fused here, real slots only) or in the tile-major
//    workspace; optionally it writes the query's log-sum-exp, m + log2 l
//    scaled back to natural log, from the same running max and row sum.
#include "mfma_util.h"

namespace sa {

namespace {

using namespace mfma;

constexpr int kWaves = 8;    // waves 0-3: first query tile of the pair, 4-7: second
constexpr int kThreads = 64 * kWaves;
constexpr int kList = 2048;  // pair-list entries staged in LDS at a time

// Real tokens of tile j.
__device__ __forceinline__ int tile_tokens(const Layout &L, const AttnParams &P, int j)
{
    return mfma::tile_tokens(L, P.div_plane, P.div_row, j);
}

// Geometry of one stage (64 keys of one key tile) in LDS: K rows [64][D] and
// transposed V [D][64], each swizzled and D KB, moved as 1 KB DMA blocks of
// 64 lanes x 16 bytes.  Wave w moves blocks [w BPW, (w + 1) BPW) of the 2 D
// blocks: the first half of the waves moves K, the second half V^T.
template <int D>
struct Stage {
    static constexpr int KBLK = kStage * D * 2 / 1024;  // K blocks (V^T has as many)
    static constexpr int BPW = 2 * KBLK / kWaves;       // blocks per wave
    static constexpr int PART = KBLK * 1024;            // bytes of K (or of V^T)
};

// Per-lane source offsets of this wave's DMA blocks.  LDS byte 16 l of a
// block receives lane l's 16 bytes, so each lane fetches the global chunk
// that the swizzle puts there.
template <int D>
struct DmaPlan {
    __amdgpu_buffer_rsrc_t rsrc;  // K of head h, or V^T of head h (N_pad D 2 bytes)
    bool is_v;                    // wave-uniform
    int off[Stage<D>::BPW];       // byte offset of the lane's chunk within a stage
};

template <int D>
__device__ __forceinline__ void make_plan(DmaPlan<D> &pl, const uint16_t *Kp, const uint16_t *Vt,
                                          const Layout &L, int h, int wave, int lane)
{
    constexpr int KBLK = Stage<D>::KBLK, BPW = Stage<D>::BPW;
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

// Byte offset of stage (key tile j, half `half`) within the head's buffer.
template <int D>
__device__ __forceinline__ int stage_offset(const DmaPlan<D> &pl, int j, int half)
{
    return pl.is_v ? (j * D * kTile + half * kStage) * 2 : (j * kTile + half * kStage) * D * 2;
}

// Issue this wave's DMA block t of a stage whose K goes to Kd and V^T to Vd.
template <int D>
__device__ __forceinline__ void issue_block(const DmaPlan<D> &pl, char *Kd, char *Vd, int soff, int wave,
                                            int t)
{
    const int blk = wave * Stage<D>::BPW + t;
    lds_char *dst = pl.is_v ? (lds_char *)Vd + (blk - Stage<D>::KBLK) * 1024 : (lds_char *)Kd + blk * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(pl.rsrc, (__attribute__((address_space(3))) void *)dst, 16,
                                             pl.off[t], soff, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_mfma_kernel(Layout L, AttnParams P)
{
    constexpr int KS = D / 16;
    constexpr int NB = D / 32;
    constexpr int BPW = Stage<D>::BPW;
    constexpr int SB = Stage<D>::PART;
    // The ring: stage slot k holds K in Kk and V^T in Vk.
    __shared__ __attribute__((aligned(1024))) char K0[SB];
    __shared__ __attribute__((aligned(1024))) char K1[SB];
    __shared__ __attribute__((aligned(1024))) char K2[SB];
    __shared__ __attribute__((aligned(1024))) char K3[SB];
    __shared__ __attribute__((aligned(1024))) char V0[SB];
    __shared__ __attribute__((aligned(1024))) char V1[SB];
    __shared__ __attribute__((aligned(1024))) char V2[SB];
    __shared__ __attribute__((aligned(1024))) char V3[SB];
    __shared__ int clist[kList];

    const uint16_t *__restrict__ Qp = (const uint16_t *)P.q;
    const uint16_t *__restrict__ Kp = (const uint16_t *)P.k;
    const uint16_t *__restrict__ Vt = (const uint16_t *)P.v;
    uint16_t *__restrict__ Op = (uint16_t *)P.o;
    const int *__restrict__ cols = P.pairs.cols;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep it scalar
    const int l32 = lane & 31, hi = lane >> 5;
    const int side = wave >> 2;  // query tile of the pair this wave serves
    const int sub = wave & 3;    // its 32-query block within that tile

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
    const int r = P.pairs.order[w];
    if (!P.pair_flag[r])
        return;  // the row kernel serves these two tiles
    const int h = r / L.nP;
    const TilePair tp = pair_tiles(L, r - h * L.nP);
    const int i = side ? tp.t2 : tp.t1;
    const int ci = i >= 0 ? tile_tokens(L, P, i) : 0;
    const bool wave_active = sub * 32 < ci;
    const int my_bit = 1 << side;

    // This lane's query: slot sub * 32 + l32 of tile i, a real token when
    // the slot is below c_i.  Its row in q and o is the raster token
    // (raster I/O, real slots only) or the tile-major slot.
    const int slot = sub * 32 + l32;
    const bool q_real = slot < ci;
    const int tok = (q_real && (P.raster || P.lse)) ? raster_token(L, i, slot) : 0;
    const long long qrow = P.raster ? (long long)h * L.N + tok
                                    : (long long)h * L.Npad + (long long)max(i, 0) * kTile + slot;
    const bool q_io = wave_active && (q_real || !P.raster);
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

    const int beg = P.pairs.row_ptr[r];
    const int end = (int)min((long long)P.pairs.row_ptr[r + 1], P.pairs.cap);

    // The pair's list entries, staged in LDS as a ring of two halves: entry
    // idx lives at clist[(idx - beg) % kList].  The first kList entries are
    // loaded up front.  When a wave's cursor reaches the middle of the k-th
    // kHalf entries (k >= 1), that wave loads its share of the next kHalf
    // entries into the other half, which every cursor has left by then
    // (cursors differ by at most one entry); hundreds of barriers pass
    // before any cursor gets there, so no barrier of its own is needed.
    constexpr int kHalf = kList / 2;
    {
        const int n = min(end - beg, kList);
        for (int u = tid; u < n; u += kThreads)
            clist[u] = cols[beg + u];
        __syncthreads();
    }
    auto refill = [&](int first) {  // entries [first, first + kHalf) of the list
        for (int u = wave * 64 + lane; u < kHalf; u += kThreads) {
            const int e = first + u;
            if (e < end)
                clist[(e - beg) & (kList - 1)] = cols[e];
        }
    };
    static_assert((kList & (kList - 1)) == 0, "ring index by mask");

    DmaPlan<D> plan;
    make_plan<D>(plan, Kp, Vt, L, h, wave, lane);

    // Stage cursor (per wave; every wave takes the same stages in the same
    // order): entry idx (packed, see pair_entry) and which 64-key half of
    // its key tile.  The entry after it is read one take ahead, so the LDS
    // latency of the list read hides behind a phase of other work.
    int idx = beg, half = 0, e_cur = 0;
    int e_next = 0;  // raw LDS read of entry idx + 1 (lanes agree)
    auto read_entry = [&](int at) {
        const int rel = at - beg;
        if (rel >= kList - kHalf / 2 && (rel & (kHalf - 1)) == kHalf / 2)
            refill(at + kHalf / 2);
        return clist[rel & (kList - 1)];
    };
    if (beg < end)
        e_cur = __builtin_amdgcn_readfirstlane(read_entry(beg));
    if (beg + 1 < end)
        e_next = read_entry(beg + 1);
    // Takes the next stage: returns its descriptor (kv | bits << 8 | 1 << 10;
    // 0 past the end) and its byte offset in this wave's buffer (K or V^T of
    // the head).  Past the end the offset is that of the head's first stage,
    // always in bounds; that copy lands in a slot nobody reads again.
    auto take = [&](int &src) -> int {
        if (idx >= end) {
            src = 0;
            return 0;
        }
        const int j = e_cur & 0xffff;
        const int c = (e_cur >> kPairCountShift) & 255;
        const int bits = (e_cur >> kPairBitsShift) & 3;
        const int kv = min(kStage, c - half * kStage);
        src = stage_offset<D>(plan, j, half);
        const int desc = kv | (bits << 8) | (1 << 10);
        if (half == 0 && c > kStage) {
            half = 1;
        } else {
            ++idx;
            half = 0;
            e_cur = __builtin_amdgcn_readfirstlane(e_next);
            if (idx + 1 < end)
                e_next = read_entry(idx + 1);
        }
        return desc;
    };
    // Per-lane LDS offsets of the MFMA operands within a stage: K chunk
    // 2 ks + hi of row key_of_mfma_row(l32), and V^T chunk 2 q + hi of row l32.
    int kofs[KS], vofs[4];
    {
        const int prow = key_of_mfma_row(l32);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kofs[ks] = lds_off<D / 8>(prow, 2 * ks + hi);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            vofs[q] = lds_off<8>(l32, 2 * q + hi);
    }

    // Ping-pong schedule.  Group A (waves 0-3, first query tile) and group B
    // (waves 4-7, second tile) share the stages; each SIMD hosts one wave of
    // each.  Step s, one workgroup barrier at its top:
    //
    //   A: [barrier] O += P V (s-1), S = K Q^T (s), copies, softmax (s)
    //   B: [barrier] copies, softmax (s-1), O += P V (s-1), S = K Q^T (s)
    //
    // so while one wave of a SIMD issues matrix products the other runs its
    // exponentials (B's scores of stage s wait in registers for its next
    // step).  Both groups read K(s) and V^T(s-1) in step s; stage t lives in
    // ring slot t % 4.  Each wave copies its share of stage s + 2 (K by group
    // A, V^T by group B, BPW blocks per wave) in step s, into the slot of
    // stage s - 2, whose K was read in step s - 2 and V^T in step s - 1.  At
    // the top of step s a wave waits for its copies of stage s (those of
    // s + 1 may still fly): K(s) is read in step s, V^T(s) in step s + 1.
    // Both groups run the same steps and leave after the same one, so they
    // pass the same barriers.
    // Descriptors: kv | bits << 8 | 1 << 10 (0: no such stage).
    int d0, d1;
    {
        int src;
        d0 = take(src);
#pragma unroll
        for (int t = 0; t < BPW; ++t)
            issue_block<D>(plan, K0, V0, src, wave, t);
        d1 = take(src);
#pragma unroll
        for (int t = 0; t < BPW; ++t)
            issue_block<D>(plan, K1, V1, src, wave, t);
    }
    auto attends = [&](int d) { return wave_active && ((d >> 8) & my_bit); };
    Scores S;
    Probs Pr;
    // Step s: K(s) in Kc, V^T(s-1) in Vp; stage s+2 is taken and copied to
    // Kn, Vn before the softmax, which has room for the scalar work and the
    // copy issue while the other group's wave keeps the matrix core busy.
    // A step returns whether stage s existed (otherwise it only finished
    // s-1).  The slots are distinct arrays addressed statically, so the
    // compiler can tell the reads of one slot from the copies in flight to
    // the others.  Each group has its own copy of the loop, so the scores
    // B keeps across the barrier and the probabilities A keeps across it do
    // not share a register allocation.
    //
    // Hide the operand offsets from loop-invariant hoisting: otherwise the
    // compiler keeps a full set of addresses per slot live across the loop
    // and runs out of registers.  Recomputing them costs one add per offset
    // per step.
    auto hide = [&]() {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            asm volatile("" : "+v"(kofs[ks]));
#pragma unroll
        for (int q = 0; q < 4; ++q)
            asm volatile("" : "+v"(vofs[q]));
    };
    auto copy = [&](char *Kn, char *Vn, int &dnext) {
        int src;
        dnext = take(src);
#pragma unroll
        for (int t = 0; t < BPW; ++t)
            issue_block<D>(plan, Kn, Vn, src, wave, t);
    };
    auto step_a = [&](const char *Kc, const char *Vp, char *Kn, char *Vn, int dprev, int dcur, int &dnext) {
        hide();
        wait_vmcnt<BPW>();
        lds_barrier();
        if (attends(dprev))
            pv_stage<D>(Vp, [&](int q) { return vofs[q]; }, Pr, dprev & 255, st);
        if (attends(dcur))
            qk_stage<D>(S, Kc, qf, [&](int ks) { return kofs[ks]; }, dcur & 255, hi);
        copy(Kn, Vn, dnext);
        if (attends(dcur))
            online_softmax<D>(Pr, S, dcur & 255, sl2, st);
        return dcur != 0;
    };
    auto step_b = [&](const char *Kc, const char *Vp, char *Kn, char *Vn, int dprev, int dcur, int &dnext) {
        hide();
        wait_vmcnt<BPW>();
        lds_barrier();
        copy(Kn, Vn, dnext);
        if (attends(dprev)) {
            online_softmax<D>(Pr, S, dprev & 255, sl2, st);
            pv_stage<D>(Vp, [&](int q) { return vofs[q]; }, Pr, dprev & 255, st);
        }
        if (attends(dcur))
            qk_stage<D>(S, Kc, qf, [&](int ks) { return kofs[ks]; }, dcur & 255, hi);
        return dcur != 0;
    };
    int dm1 = 0;
    if (side == 0) {
        for (;;) {
            int d2;
            if (!step_a(K0, V3, K2, V2, dm1, d0, d2))
                break;
            dm1 = d0, d0 = d1, d1 = d2;
            if (!step_a(K1, V0, K3, V3, dm1, d0, d2))
                break;
            dm1 = d0, d0 = d1, d1 = d2;
            if (!step_a(K2, V1, K0, V0, dm1, d0, d2))
                break;
            dm1 = d0, d0 = d1, d1 = d2;
            if (!step_a(K3, V2, K1, V1, dm1, d0, d2))
                break;
            dm1 = d0, d0 = d1, d1 = d2;
        }
    } else {
        for (;;) {
            int d2;
            if (!step_b(K0, V3, K2, V2, dm1, d0, d2))
                break;
            dm1 = d0, d0 = d1, d1 = d2;
            if (!step_b(K1, V0, K3, V3, dm1, d0, d2))
                break;
            dm1 = d0, d0 = d1, d1 = d2;
            if (!step_b(K2, V1, K0, V0, dm1, d0, d2))
                break;
            dm1 = d0, d0 = d1, d1 = d2;
            if (!step_b(K3, V2, K1, V1, dm1, d0, d2))
                break;
            dm1 = d0, d0 = d1, d1 = d2;
        }
    }
    wait_vmcnt<0>();  // no copy may land after the workgroup ends

    finish_rows<D>(st, wave_active, lse_at, q_io ? Op + qrow * D : nullptr, hi);
}

}  // namespace

hipError_t launch_attention_mfma(const Layout &L, const AttnParams &p, hipStream_t s)
{
    const dim3 grid(L.heads * L.nP);
    if (L.D == 128)
        hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, dim3(kThreads), 0, s, L, p);
    else
        hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, dim3(kThreads), 0, s, L, p);
    return hipGetLastError();
}

}  // namespace sa
