// Diagnostic: the rate at which this GPU sustains the instruction mix of one
// attention stage when nothing else is in the way.  It is measurement
// context for the attention kernels' fraction of the published matrix peak,
// not part of the attention path.
//
// Each wave runs `iters` stages of what a wave of the row kernel does per
// 64-key stage: S^T = K Q^T as 16 v_mfma_f32_32x32x16_bf16 products with K
// read from LDS, the online-softmax step of the attention kernels
// (mfma::online_softmax: scale and reference FMA, exp2, bf16 packs, v_dot2
// row sums, the wave-uniform redo test), and O^T += V^T P^T as 16 more
// products with V^T read from LDS, with workgroup barriers.  The LDS stage
// is written once before the loop, so there are no copies, no key lists and
// no global memory traffic inside it.  Two schedules:
//  - independent: workgroups of 4 waves (one per SIMD) run W to a compute
//    unit, so each SIMD holds W unsynchronised waves; W = 2 is the row
//    kernel's occupancy, W = 3 one wave more than any attention kernel
//    holds; as in the row kernel, one barrier per stage, operands read
//    inline, issue priority raised for the softmax;
//  - ping-pong: one workgroup of 8 waves per compute unit, two per SIMD, in
//    the pair kernel's schedule, one barrier per step: waves 0-3 run
//    O^T += V^T P^T (previous stage), S^T = K Q^T, then the softmax; waves
//    4-7 the softmax of the previous stage, then their products; so while
//    one wave of a SIMD issues products the other runs its softmax.  The
//    products are the pair kernel's own (mfma::qk_stage, mfma::pv_stage).
//
// Operands are pseudo-random bf16 values in [-1, 1) (an integer hash of
// their position), so the matrix cores switch about as much as with real
// activations; the clock, and with it the rate, depends on that power.
#include "mix_probe.h"

#include "mfma_util.h"

namespace sa {

namespace {

using namespace mfma;

constexpr int kD = 128;
constexpr int kStageBytes = 2 * kStage * kD * 2;  // K [64][128] then V^T [128][64], bf16

// A value in [-1, 1) from a 32-bit position (lowbias32 integer hash).
__device__ __forceinline__ float hash_unit(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return (float)(int32_t)x * (1.0f / 2147483648.0f);
}

// A workgroup barrier that no instruction is scheduled across, so each
// phase holds exactly its own work (in the attention kernels the phases are
// separate conditional blocks, which has the same effect).
__device__ __forceinline__ void fenced_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void zero_scores(Scores &S)
{
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
        S.s0[jj] = 0.f;
        S.s1[jj] = 0.f;
    }
}

// Operands and state of one wave: Q in registers, the running softmax state,
// and the per-lane LDS offsets of the K and V^T operands of a stage.
struct ProbeWave {
    bf16x8 qf[kD / 16];
    RowState<kD> st;
    int kofs[kD / 16], vofs[4];
    int prow;
};

__device__ __forceinline__ void init_wave(ProbeWave &w, uint32_t seed, int l32, int hi)
{
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
#pragma unroll
        for (int u = 0; u < 8; ++u)
            w.qf[ks][u] = (__bf16)hash_unit(0x85ebca6bu * seed + 8 * ks + u);
#pragma unroll
    for (int nb = 0; nb < kD / 32; ++nb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            w.st.acc[nb][jj] = 0.f;
    w.st.m = -INFINITY;
    w.st.l = 0.f;
    w.prow = key_of_mfma_row(l32);
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
        w.kofs[ks] = lds_off<kD / 8>(w.prow, 2 * ks + hi);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        w.vofs[q] = lds_off<8>(l32, 2 * q + hi);
}

__device__ __forceinline__ void fill_stage(char *stage, int tid, int threads)
{
    for (int i = tid; i < kStageBytes / 2; i += threads)
        ((__bf16 *)stage)[i] = (__bf16)hash_unit(0x9e3779b9u * blockIdx.x + i);
    __syncthreads();
}

__device__ __forceinline__ float wave_sum(const ProbeWave &w)
{
    float s = w.st.l;
#pragma unroll
    for (int nb = 0; nb < kD / 32; ++nb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            s += w.st.acc[nb][jj];
    return s;
}

// The row kernel's schedule: one barrier per stage, operands read inline
// (the compiler schedules them), issue priority raised for the softmax.
template <int W>
__global__ __launch_bounds__(256, W) void mix_kernel(int iters, long long *cycles, float *sink)
{
    constexpr int KS = kD / 16, NB = kD / 32, RCK = kD / 8;
    __shared__ __attribute__((aligned(1024))) char stage[kStageBytes];
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    fill_stage(stage, tid, 256);
    ProbeWave w;
    init_wave(w, blockIdx.x * 256 + tid, l32, hi);
    const float sl2 = 1.4426950408889634f / sqrtf((float)kD);
    const char *Ks = stage, *Vs = stage + kStageBytes / 2;

    const long long t0 = (long long)__builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
        fenced_barrier();
        Scores S;
        zero_scores(S);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a0 = *(const bf16x8 *)(Ks + lds_off<RCK>(w.prow, 2 * ks + hi));
            const bf16x8 a1 = *(const bf16x8 *)(Ks + lds_off<RCK>(32 + w.prow, 2 * ks + hi));
            S.s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, w.qf[ks], S.s0, 0, 0, 0);
            S.s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, w.qf[ks], S.s1, 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(2);
        Probs P;
        online_softmax<kD>(P, S, kStage, sl2, w.st);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                w.st.acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    *(const bf16x8 *)(Vs + lds_off<8>(32 * nb + l32, 2 * q + hi)), P.p[q], w.st.acc[nb], 0, 0, 0);
    }
    fenced_barrier();
    const long long t1 = (long long)__builtin_amdgcn_s_memtime();
    sink[blockIdx.x * 256 + tid] = wave_sum(w);
    if (lane == 0)
        cycles[blockIdx.x * 4 + (tid >> 6)] = t1 - t0;
}

// The pair kernel's ping-pong: 8 waves, one barrier per step; waves 0-3 run
// products then softmax, waves 4-7 the previous stage's softmax then their
// products.
__global__ __launch_bounds__(512, 1) void mix_pingpong_kernel(int iters, long long *cycles, float *sink)
{
    __shared__ __attribute__((aligned(1024))) char stage[kStageBytes];
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int group = __builtin_amdgcn_readfirstlane(tid >> 8);
    fill_stage(stage, tid, 512);
    ProbeWave w;
    init_wave(w, blockIdx.x * 512 + tid, l32, hi);
    const float sl2 = 1.4426950408889634f / sqrtf((float)kD);
    const char *Ks = stage, *Vs = stage + kStageBytes / 2;
    Probs P;
    Scores S;

    const long long t0 = (long long)__builtin_amdgcn_s_memtime();
    if (group == 0) {
        for (int it = 0; it < iters; ++it) {
            fenced_barrier();
            if (it > 0)
                pv_stage<kD>(Vs, [&](int q) { return w.vofs[q]; }, P, kStage, w.st);
            qk_stage<kD>(S, Ks, w.qf, [&](int ks) { return w.kofs[ks]; }, kStage, hi);
            online_softmax<kD>(P, S, kStage, sl2, w.st);
        }
        fenced_barrier();
        pv_stage<kD>(Vs, [&](int q) { return w.vofs[q]; }, P, kStage, w.st);
    } else {
        for (int it = 0; it < iters; ++it) {
            fenced_barrier();
            if (it > 0) {
                online_softmax<kD>(P, S, kStage, sl2, w.st);
                pv_stage<kD>(Vs, [&](int q) { return w.vofs[q]; }, P, kStage, w.st);
            }
            qk_stage<kD>(S, Ks, w.qf, [&](int ks) { return w.kofs[ks]; }, kStage, hi);
        }
        fenced_barrier();  // both groups pass iters + 1 barriers
        online_softmax<kD>(P, S, kStage, sl2, w.st);
        pv_stage<kD>(Vs, [&](int q) { return w.vofs[q]; }, P, kStage, w.st);
    }
    const long long t1 = (long long)__builtin_amdgcn_s_memtime();
    sink[blockIdx.x * 512 + tid] = wave_sum(w);
    if (lane == 0)
        cycles[blockIdx.x * 8 + (tid >> 6)] = t1 - t0;
}

}  // namespace

hipError_t launch_mix_probe(int waves_per_simd, int pingpong, int cus, int iters, long long *cycles, float *sink,
                            hipStream_t s)
{
    if (pingpong) {
        hipLaunchKernelGGL(mix_pingpong_kernel, dim3(cus), dim3(512), 0, s, iters, cycles, sink);
        return hipGetLastError();
    }
    const dim3 grid(cus * waves_per_simd), block(256);
    if (waves_per_simd == 1)
        hipLaunchKernelGGL(mix_kernel<1>, grid, block, 0, s, iters, cycles, sink);
    else if (waves_per_simd == 2)
        hipLaunchKernelGGL(mix_kernel<2>, grid, block, 0, s, iters, cycles, sink);
    else
        hipLaunchKernelGGL(mix_kernel<3>, grid, block, 0, s, iters, cycles, sink);
    return hipGetLastError();
}

}  // namespace sa
