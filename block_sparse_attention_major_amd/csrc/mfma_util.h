// Device helpers shared by the bf16 matrix-core kernels (the pair and row
// attention kernels and the tile-mass kernel): vector types, the swizzled
// LDS tile layout, the MFMA key order, wait/barrier helpers, the per-wave
// softmax state and the online-softmax step.
//
// All of it serves S^T = K Q^T on v_mfma_f32_32x32x16_bf16: a wave holds 32
// queries, lane l owns query l % 32, and lanes l and l ^ 32 hold the two
// halves of that query's keys, so row reductions are in-lane plus one
// v_permlane32_swap.
#pragma once

#include "common.h"

namespace sa {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kTile = 128;   // slots per tile
constexpr int kStage = 64;   // keys per LDS stage (half a tile)

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

// Lanes l and l ^ 32 hold the two halves of one query row.
__device__ __forceinline__ float half_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// acc + sum of the 8 bf16 values of p (two per v_dot2 with a vector of ones).
__device__ __forceinline__ float row_sum_bf16(bf16x8 p, float acc)
{
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
}

// Real tokens of tile j (clipped at the far edges of the grid); the
// divisions by tiles per plane and per row go through fixed-divisor
// multiplies.
__device__ __forceinline__ int tile_tokens(const Layout &L, const FastDiv &div_plane, const FastDiv &div_row,
                                           int j)
{
    const int a = (int)fast_div((uint32_t)j, div_plane);
    const int rem = j - a * L.ny * L.nx;
    const int b = (int)fast_div((uint32_t)rem, div_row);
    const int e = rem - b * L.nx;
    return min(L.tt, L.T - a * L.tt) * min(L.th, L.H - b * L.th) * min(L.tw, L.W - e * L.tw);
}

// Copies of K and V^T into LDS move 1 KB blocks: lane l of a
// buffer_load ... lds writes LDS bytes 16 l .. 16 l + 15 of the block, so
// each lane fetches the global chunk that the LDS layout puts there.
// Block kb of K rows (D / 8 chunks per row, lds_off<D / 8>) holds 256-byte
// lines 4 kb .. 4 kb + 3; this is the byte offset, from the first row, of
// the K chunk lane `lane` copies for it.
template <int D>
__device__ __forceinline__ int k_chunk_src(int kb, int lane)
{
    constexpr int RC = D / 8, RPL = 16 / RC;
    const int line = 4 * kb + (lane >> 4);
    const int logical = (lane & 15) ^ (line & 15);
    const int row = RPL * line + logical / RC, c = logical % RC;
    return row * D * 2 + 16 * c;
}
// The same for block kb of a 64-key stage of V^T (rows of 64 keys,
// lds_off<8>), copied from the per-tile [D][kTile] layout: the byte offset
// from the stage's first key of feature row 0.
__device__ __forceinline__ int vt_chunk_src(int kb, int lane)
{
    const int line = 4 * kb + (lane >> 4);
    const int logical = (lane & 15) ^ (line & 15);
    const int dv = 2 * line + (logical >> 3), c = logical & 7;
    return dv * kTile * 2 + 16 * c;
}

// s_waitcnt on this wave's vector-memory counter only (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that waits for this wave's LDS operations but leaves its
// DMA copies in flight (__syncthreads would drain those as well).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
}

// The per-wave state of one query block: 32 queries x D features, O^T
// accumulated with one query per lane.
template <int D>
struct RowState {
    f32x16 acc[D / 32];
    float m, l;  // running max (log2 units) and partial row sum of this lane
};

// Scores of a wave's 32 queries against the keys of one 64-key stage, as
// two 32-key halves (result register j of lane l: key 16 (j / 8) +
// 8 (l / 32) + j % 8 of the half, query l % 32).
struct Scores {
    f32x16 s0, s1;
};
// Probabilities in bf16, in the B-operand order of O^T += V^T P^T: 16-key
// steps 0..3 of the stage.
struct Probs {
    bf16x8 p[4];
};

// A lane's probability sum for one stage may reach kProbCap before the
// stage is redone against its true maximum (see online_softmax).
constexpr float kProbCap = 65536.0f;

// Probabilities of 16-key step q (0..3) of a stage against the reference m,
// rounded to bf16 into P.p[q]; returns ls plus their sum.  The steps are
// summed in order, so a stage's row sum is the same however its steps are
// split between calls.
__device__ __forceinline__ float step_probs(Probs &P, const Scores &S, int q, float sl2, float m, float ls)
{
    const f32x16 &src = q < 2 ? S.s0 : S.s1;
    const int o = (q & 1) * 8;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
        P.p[q][jj] = (__bf16)exp2_fast(fmaf(src[o + jj], sl2, -m));
    return row_sum_bf16(P.p[q], ls);
}

// The redo of a stage whose probability sum left [0, kProbCap]: moves the
// reference to the true running maximum, rescales the accumulator and row
// sum, and recomputes the stage's probabilities; returns their sum.
template <int D>
__device__ __forceinline__ float redo_stage(Probs &P, const Scores &S, bool two, float sl2, RowState<D> &st)
{
    constexpr int NB = D / 32;
    float mx = S.s0[0];
#pragma unroll
    for (int jj = 1; jj < 16; ++jj)
        mx = fmaxf(mx, S.s0[jj]);
    if (two) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            mx = fmaxf(mx, S.s1[jj]);
    }
    const float t = half_max(mx) * sl2;
    const float m_new = fmaxf(st.m, t);
    const float alpha = exp2_fast(st.m - m_new);
    st.m = m_new;
    st.l *= alpha;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            st.acc[nb][jj] *= alpha;
    float ls = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (q < 2 || two)
            ls = step_probs(P, S, q, sl2, st.m, ls);
    return ls;
}

// Online softmax step over the kv real keys (1..64) of a stage: scores ->
// bf16 probabilities, running row sum updated, accumulator rescaled when the
// reference moves.  sl2 = softmax scale * log2(e).
//
// The probabilities are first taken against the running reference st.m as
// it stands (no row maximum), and the stage is redone only when a lane's sum
// of them leaves [0, kProbCap]: on the first stage (st.m = -inf gives
// inf or NaN) or when a score exceeds the reference by about 11 or more in
// log2 units.  The redo moves the reference to the true running maximum
// (computed then), rescales the accumulator and row sum by 2^(old - new),
// and recomputes the probabilities; that branch is wave-uniform.  Numerator
// and denominator share the reference, so the result does not depend on
// it; each probability stays at or below kProbCap.
template <int D>
__device__ __forceinline__ void online_softmax(Probs &P, const Scores &S, int kv, float sl2, RowState<D> &st)
{
    const bool two = kv > 32;
    float ls = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (q < 2 || two)
            ls = step_probs(P, S, q, sl2, st.m, ls);
    if (__ballot(!(ls <= kProbCap)))
        ls = redo_stage<D>(P, S, two, sl2, st);
    st.l += ls;
}

// Keys past kv (1..63) of a stage score -inf: key 16 (jj / 8) + 8 hi +
// jj % 8 of each half is past the end when 16 (jj / 8) + jj % 8 >= kv - 8 hi.
__device__ __forceinline__ void mask_stage_tail(Scores &S, int kv, int hi)
{
    const int lim = kv - 8 * hi;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
        const int c = 16 * (jj >> 3) + (jj & 7);
        if (c >= lim)
            S.s0[jj] = -INFINITY;
        if (32 + c >= lim)
            S.s1[jj] = -INFINITY;
    }
}

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMFMA = 0x008, kSchedDSRead = 0x100;

// S = K Q^T for the kv real keys (1..64) of the stage whose K is at Ks;
// kofs(ks) is the lane's operand offset for k-step ks,
// lds_off<D / 8>(key_of_mfma_row(l32), 2 ks + hi) (which is that of k-step 0
// XOR ks << 5).  Keys past kv score -inf.  Operands are read two k-steps
// ahead of the products that use them, so the LDS latency hides behind four
// matrix instructions.
template <int D, typename KOfs>
__device__ __forceinline__ void qk_stage(Scores &S, const char *Ks, const bf16x8 (&qf)[D / 16], KOfs &&kofs,
                                         int kv, int hi)
{
    constexpr int KS = D / 16;
    constexpr int SUB1 = 64 * D;  // second 32-key half: 32 rows further on, same swizzle
    const bool two = kv > 32;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
        S.s0[jj] = 0.f;
        S.s1[jj] = 0.f;
    }
    if (two) {
        bf16x8 r0[KS], r1[KS];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            r0[ks] = *(const bf16x8 *)(Ks + kofs(ks));
            r1[ks] = *(const bf16x8 *)(Ks + SUB1 + kofs(ks));
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS) {
                r0[ks + 2] = *(const bf16x8 *)(Ks + kofs(ks + 2));
                r1[ks + 2] = *(const bf16x8 *)(Ks + SUB1 + kofs(ks + 2));
            }
            S.s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r0[ks], qf[ks], S.s0, 0, 0, 0);
            S.s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r1[ks], qf[ks], S.s1, 0, 0, 0);
        }
        // Keep that order: reads of steps 0 and 1, then per step the reads
        // of step ks + 2 and the products of ks.
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 4, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS)
                __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 2, 0);
        }
    } else {
        bf16x8 r0[KS];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            r0[ks] = *(const bf16x8 *)(Ks + kofs(ks));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS)
                r0[ks + 2] = *(const bf16x8 *)(Ks + kofs(ks + 2));
            S.s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r0[ks], qf[ks], S.s0, 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS)
                __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        }
    }
    if (kv < kStage)
        mask_stage_tail(S, kv, hi);
}

// O^T += V^T P^T over the stage whose V^T is at Vs (kv real keys); vofs(q)
// is the lane's operand offset for 16-key step q, lds_off<8>(l32, 2 q + hi)
// (that of step 0 XOR q << 5).  The operands of key step q + 1 are read
// while the products of step q run.
template <int D, typename VOfs>
__device__ __forceinline__ void pv_stage(const char *Vs, VOfs &&vofs, const Probs &P, int kv, RowState<D> &st)
{
    constexpr int NB = D / 32;
    const int steps = kv > 32 ? 4 : 2;
    // A operand = V^T rows 32 nb + l32, keys in 16-key steps (rows 32 apart
    // are 16 swizzle lines apart: same pattern, 4 KB on).
    bf16x8 va[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        va[nb] = *(const bf16x8 *)(Vs + 4096 * nb + vofs(0));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (q < steps) {
            bf16x8 vn[NB];
            if (q + 1 < steps) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    vn[nb] = *(const bf16x8 *)(Vs + 4096 * nb + vofs(q + 1));
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                st.acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[nb], P.p[q], st.acc[nb], 0, 0, 0);
            if (q + 1 < steps) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    va[nb] = vn[nb];
            }
        }
    }
    if (steps == 4) {
        // Keep that order: reads of step q + 1, then the products of q.
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, NB, 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q + 1 < 4)
                __builtin_amdgcn_sched_group_barrier(kSchedDSRead, NB, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, NB, 0);
        }
    }
}

// Epilogue of a wave: normalizes the accumulator by the row sum (both lane
// halves), writes the query's log-sum-exp (natural log; -inf for an empty
// row) when lse_at is set, and its O row (bf16) when orow is set.  Every
// lane of the wave must call it (half_sum exchanges lanes l and l ^ 32).
template <int D>
__device__ __forceinline__ void finish_rows(const RowState<D> &st, bool active, float *lse_at, uint16_t *orow,
                                            int hi)
{
    constexpr int NB = D / 32;
    const float lt = active ? half_sum(st.l) : 0.f;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // st.m is in log2 units and st.l sums exp2(score * log2 e - st.m).
    if (lse_at)
        *lse_at = lt > 0.f ? (st.m + log2f(lt)) * kLn2 : -INFINITY;
    if (orow) {
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
                    pk.b[u] = (__bf16)(st.acc[nb][4 * g + u] * inv);
                *(uint2 *)(orow + 32 * nb + 8 * g + 4 * hi) = pk.u;
            }
        }
    }
}

}  // namespace mfma
}  // namespace sa
