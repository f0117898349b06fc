// ttt_linear_combine.hip -- start states of the segments of a segmented
// TTT-Linear scan, with or without momentum.
//
// A chunk of the scan maps the fast weights affinely,
//     W' = (I - eta K^T K) W + eta K^T V
// (mini-batch gradient descent on 1/2 ||K W - V||^2 with all gradients at the
// chunk-start W: "Test-Time Training Layers: How Inner-Loop Gradient Descent
// Replaces the Transformer KV Cache ...", sections "The Core Mechanism" and
// "Hardware Parallelization"), so a segment of chunks does too:
// W_end = M W_start + N.  With momentum (the E2-TTT write-up on zhichai.net,
// section "Core Math") a chunk maps the pair X = [W; M] (2d rows) affinely in
// the same way, column by column.  Given the maps (M_j, N_j) of segments
// 0 .. nseg - 2 (M_j of kRows x kRows, N_j of kRows x d), this kernel computes
//     X_0 = [W0; M0],   X_{j+1} = M_j X_j + N_j
// and stores every X_j.  The segments then run their scans independently.
//
// Column j of X_{j+1} depends only on column j of X_j, so one chain is split
// over 4 workgroups, one per 16-column slice J (all on the XCD of the chain's
// maps and scans); wave I of a workgroup computes
// the 16 x 16 output tile (I, J) of each step in fp32 on
// v_mfma_f32_16x16x4_f32 (kRows / 4 k-steps in 4 independent accumulators).
// Every slice X_j stays in LDS (rows padded to 17 floats, so the four rows
// kRows / 4 g + s a wave reads per k-step fall in different banks) and goes to
// memory at the end, so the only memory operations inside the loop are the
// loads of the M and N operands, kDepth steps ahead in a ring of register
// sets: the maps were just written by other CUs, so each load costs a trip to
// memory.
#include "ttt_internal.h"

namespace ttt {
namespace {

constexpr int kD = 64;
constexpr int kSlice = 16;
constexpr int kPad = kSlice + 1;

template <int kRows>
struct Shape {
    static constexpr int kWaves = kRows / 16;          // one row tile each
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kSliceFloats = kRows * kPad;
    static constexpr int kK = kRows / 4;               // k-steps per product (k-slot g: column kK g + s)
    static constexpr int kDepth = kRows == 64 ? 6 : 3; // steps of operands in flight
    static constexpr int64_t kMapFloats = static_cast<int64_t>(kRows) * kRows + kRows * kD;
};

template <int kRows>
size_t combine_lds_bytes(int nseg)
{
    using S = Shape<kRows>;
    return static_cast<size_t>(nseg + S::kDepth) * S::kSliceFloats * 4;
}

}  // namespace

// LDS of one combine workgroup for a chain of nseg segments (kDepth spare
// slots beyond the nseg start states)
size_t linear_combine_lds_bytes(int nseg) { return combine_lds_bytes<64>(nseg); }
size_t momentum_combine_lds_bytes(int nseg) { return combine_lds_bytes<128>(nseg); }

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// X_0 = [W0; M0] (rows kD .. kRows - 1 from M0 when kRows > kD; zero without
// M0), then the composition; xstart: [units][nseg][kRows][kD].  first = 1:
// X_1 is already in xstart (segment 0 was scanned; map 0 is not used) and
// the composition starts there.
template <int kRows>
__device__ __forceinline__ void combine_chain(const float* W0, int w0_per_batch, const float* M0,
                                              int H, int64_t units, const float* __restrict__ maps,
                                              int nseg, float* __restrict__ xstart, int first)
{
    using S = Shape<kRows>;
    constexpr int kDepth = S::kDepth;
    constexpr int kK = S::kK;
    extern __shared__ float Wl[];        // [nseg][kRows][kPad]: slice J of X_0 .. X_{nseg-1}

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
    const float* m0 = M0 ? M0 + u * kD * kD : nullptr;
    float* out = xstart + u * nseg * kRows * kD;
    const float* chain_maps = maps + u * (nseg - 1) * S::kMapFloats;

    // thread tid moves rows tid / 16 + (kRows / 4) q, column tid % 16 of a slice
    {
        float x[4];
        const float* x1 = out + kRows * kD;      // X_1 when first = 1
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = tid / 16 + (kRows / 4) * q;
            x[q] = first ? x1[row * kD + 16 * J + tid % 16]
                 : row < kD ? w0[row * kD + 16 * J + tid % 16]
                            : (m0 ? m0[(row - kD) * kD + 16 * J + tid % 16] : 0.f);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            Wl[first * S::kSliceFloats + (tid / 16 + (kRows / 4) * q) * kPad + tid % 16] = x[q];
    }

    // operands of step j: a[s] = M_j[16 I + c][kK g + s] (A of k-step s, whose
    // k-slot g is row kK g + s of X_j: one contiguous run of M per lane) and
    // n[r] = N_j[16 I + 4 g + r][16 J + c] (the accumulator's start value);
    // steps past the last one reload the last map (results unused)
    f32x4 a[kDepth][kK / 4];
    f32x4 n[kDepth];
    auto load_ops = [&](f32x4 (&dst)[kK / 4], f32x4& ndst, int j) {
        const float* M = chain_maps + min(j, nseg - 2) * S::kMapFloats;
        const float* N = M + kRows * kRows;
#pragma unroll
        for (int x = 0; x < kK / 4; ++x)
            dst[x] = *reinterpret_cast<const f32x4*>(M + (16 * I + c) * kRows + kK * g + 4 * x);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            ndst[r] = N[(16 * I + 4 * g + r) * kD + 16 * J + c];
    };
#pragma unroll
    for (int q = 0; q < kDepth; ++q)
        load_ops(a[q], n[q], first + q);     // nseg >= 2 whenever this kernel runs
    __syncthreads();

    // step j with the operands of ring entry q: X_{j+1} slice into LDS, then
    // the ring entry reloaded for step j + kDepth
    auto step = [&](int q, int j) {
        const float* Wc = Wl + j * S::kSliceFloats;
        float b[kK];
#pragma unroll
        for (int s = 0; s < kK; ++s)
            b[s] = Wc[(kK * g + s) * kPad + c];
        f32x4 acc[4] = {n[q], {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < kK; ++s)
            acc[s & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q][s >> 2][s & 3], b[s], acc[s & 3],
                                                              0, 0, 0);
        const f32x4 res = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        float* Wn = Wl + (j + 1) * S::kSliceFloats;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Wn[(16 * I + 4 * g + r) * kPad + c] = res[r];
        load_ops(a[q], n[q], j + kDepth);
        __syncthreads();
    };
    // full rounds of kDepth steps, then the last partial round with an exit
    // (kept out of the full rounds, whose schedule it would disturb)
    int j0 = first;
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

    for (int j = first; j < nseg; ++j) {
        const float* Ws = Wl + j * S::kSliceFloats;
        float* o = out + j * kRows * kD;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[(tid / 16 + (kRows / 4) * q) * kD + 16 * J + tid % 16] =
                Ws[(tid / 16 + (kRows / 4) * q) * kPad + tid % 16];
    }
}

__global__ void __launch_bounds__(Shape<64>::kThreads, 1)
linear_combine_kernel(const float* W0, int w0_per_batch, int H, int64_t units,
                      const float* __restrict__ maps, int nseg, float* __restrict__ wstart,
                      int first)
{
    combine_chain<64>(W0, w0_per_batch, nullptr, H, units, maps, nseg, wstart, first);
}

__global__ void __launch_bounds__(Shape<128>::kThreads, 1)
momentum_combine_kernel(const float* W0, int w0_per_batch, const float* M0, int H, int64_t units,
                        const float* __restrict__ maps, int nseg, float* __restrict__ xstart)
{
    combine_chain<128>(W0, w0_per_batch, M0, H, units, maps, nseg, xstart, 0);
}

template <int kRows, typename Kernel, typename... Args>
hipError_t launch_combine(Kernel kernel, int64_t units, int nseg, hipStream_t stream, Args... args)
{
    const size_t lds = combine_lds_bytes<kRows>(nseg);
    if (lds > static_cast<size_t>(kMaxLdsBytes))
        return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(lds));
        if (e != hipSuccess)
            return e;
    }
    const int64_t blocks = units < 8 ? 4 * units : 32 * ((units + 7) / 8);
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(Shape<kRows>::kThreads),
                       lds, stream, args...);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_combine(const LinearArgs& a, const SegmentPlan& p)
{
    const int64_t units = a.B * a.H;
    return launch_combine<64>(linear_combine_kernel, units, p.nseg, a.stream, a.W0,
                              a.w0_per_batch, static_cast<int>(a.H), units,
                              static_cast<const float*>(p.maps), p.nseg, p.wstart,
                              p.fused ? 1 : 0);
}

hipError_t launch_momentum_combine(const MomentumArgs& a, const float* maps, int nseg,
                                   float* xstart)
{
    const int64_t units = a.B * a.H;
    return launch_combine<128>(momentum_combine_kernel, units, nseg, a.stream, a.W0,
                               a.w0_per_batch, a.M0, static_cast<int>(a.H), units, maps, nseg,
                               xstart);
}

}  // namespace ttt
