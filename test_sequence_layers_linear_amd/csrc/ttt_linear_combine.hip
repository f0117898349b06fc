// ttt_linear_combine.hip -- start states of the segments of a segmented
// TTT-Linear scan.
//
// A chunk of the scan maps the fast weights affinely,
//     W' = (I - eta K^T K) W + eta K^T V
// (mini-batch gradient descent on 1/2 ||K W - V||^2 with all gradients at the
// chunk-start W: "Test-Time Training Layers: How Inner-Loop Gradient Descent
// Replaces the Transformer KV Cache ...", sections "The Core Mechanism" and
// "Hardware Parallelization"), so a segment of chunks does too:
// W_end = M W_start + N.  Given the maps (M_j, N_j) of segments
// 0 .. nseg - 2, this kernel computes
//     W_0 = W0,   W_{j+1} = M_j W_j + N_j
// and stores every W_j.  The segments then run their scans independently.
//
// Column j of W_{j+1} depends only on column j of W_j, so one chain is split
// over 4 workgroups, one per 16-column slice J (all on the XCD of the chain's
// maps and scans); wave I of a workgroup computes
// the 16 x 16 output tile (I, J) of each step in fp32 on
// v_mfma_f32_16x16x4_f32 (16 k-steps in 4 independent accumulators).  Every
// slice W_j stays in LDS (rows padded to 17 floats, so the four rows 16 g + s
// a wave reads per k-step fall in different banks) and goes to memory at the end, so
// the only memory operations inside the loop are the loads of the M and N
// operands, kDepth steps ahead in a ring of register sets: the maps were just
// written by other CUs, so each load costs a trip to memory.
#include "ttt_internal.h"

namespace ttt {
namespace {

constexpr int kD = 64;
constexpr int kSlice = 16;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPad = kSlice + 1;
constexpr int kSliceFloats = kD * kPad;
constexpr int kDepth = 6;                // steps of operands in flight

}  // namespace

// LDS of one combine workgroup for a chain of nseg segments (kDepth spare
// slots beyond the nseg start states)
size_t linear_combine_lds_bytes(int nseg)
{
    return static_cast<size_t>(nseg + kDepth) * kSliceFloats * 4;
}

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kThreads, 1)
linear_combine_kernel(const float* W0, int w0_per_batch, int H, int64_t units,
                      const float* __restrict__ maps, int nseg, float* __restrict__ wstart)
{
    extern __shared__ float Wl[];        // [nseg][64][kPad]: slice J of W_0 .. W_{nseg-1}

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int I = tid >> 6;              // row tile of this wave
    const int c = lane & 15;
    const int g = lane >> 4;

    // chain u and column slice J; with at least 8 chains the 4 workgroups of
    // chain u run on XCD u % 8 (workgroups go to the XCDs round robin), where
    // its maps were written
    int64_t u;
    int J;
    if (units < 8) {
        u = blockIdx.x >> 2;
        J = blockIdx.x & 3;
    } else {
        const int t = blockIdx.x >> 3;
        u = 8 * static_cast<int64_t>(t >> 2) + (blockIdx.x & 7);
        J = t & 3;
    }
    if (u >= units)
        return;
    const int h = static_cast<int>(u % H);
    const float* w0 = W0 + (w0_per_batch ? u : h) * kD * kD;
    float* out = wstart + u * nseg * kD * kD;
    const float* chain_maps = maps + u * (nseg - 1) * 2 * kD * kD;

    // thread tid moves rows tid / 16 + 16 q, column tid % 16 of a slice
    {
        float x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            x[q] = w0[(tid / 16 + 16 * q) * kD + 16 * J + tid % 16];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            Wl[(tid / 16 + 16 * q) * kPad + tid % 16] = x[q];
    }

    // operands of step j: a[s] = M_j[16 I + c][16 g + s] (A of k-step s, whose
    // k-slot g is row 16 g + s of W_j: one contiguous 64-byte run of M per
    // lane) and n[r] = N_j[16 I + 4 g + r][16 J + c] (the accumulator's start
    // value); steps past the last one reload the last map (results unused)
    f32x4 a[kDepth][4];
    f32x4 n[kDepth];
    auto load_ops = [&](f32x4 (&dst)[4], f32x4& ndst, int j) {
        const float* M = chain_maps + min(j, nseg - 2) * 2 * kD * kD;
        const float* N = M + kD * kD;
#pragma unroll
        for (int x = 0; x < 4; ++x)
            dst[x] = *reinterpret_cast<const f32x4*>(M + (16 * I + c) * kD + 16 * g + 4 * x);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            ndst[r] = N[(16 * I + 4 * g + r) * kD + 16 * J + c];
    };
#pragma unroll
    for (int q = 0; q < kDepth; ++q)
        load_ops(a[q], n[q], q);             // nseg >= 2 whenever this kernel runs
    __syncthreads();

    // step j with the operands of ring entry q: W_{j+1} slice into LDS, then
    // the ring entry reloaded for step j + kDepth
    auto step = [&](int q, int j) {
        const float* Wc = Wl + j * kSliceFloats;
        float b[16];
#pragma unroll
        for (int s = 0; s < 16; ++s)
            b[s] = Wc[(16 * g + s) * kPad + c];
        f32x4 acc[4] = {n[q], {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < 16; ++s)
            acc[s & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q][s >> 2][s & 3], b[s], acc[s & 3],
                                                              0, 0, 0);
        const f32x4 res = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        float* Wn = Wl + (j + 1) * kSliceFloats;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Wn[(16 * I + 4 * g + r) * kPad + c] = res[r];
        load_ops(a[q], n[q], j + kDepth);
        __syncthreads();
    };
    // full rounds of kDepth steps, then the last partial round with an exit
    // (kept out of the full rounds, whose schedule it would disturb)
    int j0 = 0;
    for (; j0 + kDepth + 1 <= nseg; j0 += kDepth) {
#pragma unroll
        for (int q = 0; q < kDepth; ++q)
            step(q, j0 + q);
    }
#pragma unroll
    for (int q = 0; q < kDepth; ++q) {
        if (j0 + q + 1 >= nseg)          // uniform: every start state is done
            break;
        step(q, j0 + q);
    }

    for (int j = 0; j < nseg; ++j) {
        const float* Ws = Wl + j * kSliceFloats;
        float* o = out + j * kD * kD;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[(tid / 16 + 16 * q) * kD + 16 * J + tid % 16] = Ws[(tid / 16 + 16 * q) * kPad + tid % 16];
    }
}

}  // namespace

hipError_t launch_linear_combine(const LinearArgs& a, const SegmentPlan& p)
{
    const size_t lds = linear_combine_lds_bytes(p.nseg);
    if (lds > static_cast<size_t>(kMaxLdsBytes))
        return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(linear_combine_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(lds));
        if (e != hipSuccess)
            return e;
    }
    const int64_t units = a.B * a.H;
    const int64_t blocks = units < 8 ? 4 * units : 32 * ((units + 7) / 8);
    hipLaunchKernelGGL(linear_combine_kernel, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), lds, a.stream, a.W0, a.w0_per_batch, static_cast<int>(a.H), units,
                       p.maps, p.nseg, p.wstart);
    return hipGetLastError();
}

}  // namespace ttt
