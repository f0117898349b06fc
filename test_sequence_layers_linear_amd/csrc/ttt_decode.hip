// ttt_decode.hip -- single-token TTT-Linear step (online gradient descent):
//     r = k W - v;   W <- W - eta k^T r;   y = q W (updated)
// ("Test-Time Training Layers: How Inner-Loop Gradient Descent Replaces the
// Transformer KV Cache ...", section "The Core Mechanism", steps 1-3; its
// section "Hardware Parallelization" names this sequential form as the one
// for token-by-token decoding with O(1) step cost).
//
// The step is HBM-bound on the fp32 state (read + write d*d*4 bytes per
// (batch, head)).  Output columns of W are independent (column j needs only
// W[:, j], k, q and v_j), so each (batch, head) is split over d/16 workgroups
// of 16 columns; this gives B*H*d/16 workgroups instead of B*H.  Inside a
// workgroup 16 row groups x 16 columns of threads: each thread owns d/16
// rows of one column, loads them once, and writes them back once.
//
// y_j uses q W'_j = q W_j - eta (q . k) r_j, algebraically the readout with
// the updated column, so W is read once and written once.
#include "ttt_internal.h"

namespace ttt {
namespace {

constexpr int kCols = 16;
constexpr int kRowGroups = 16;

template <typename TIn>
__global__ void __launch_bounds__(kCols * kRowGroups)
decode_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
              const TIn* __restrict__ v, float* __restrict__ W,
              const float* __restrict__ eta, int H, int d, TIn* __restrict__ y)
{
    __shared__ float ks[128], qs[128];
    __shared__ float red_k[kRowGroups][kCols + 1], red_q[kRowGroups][kCols + 1];
    __shared__ float rcol[kCols];
    __shared__ float qk_s;

    const int64_t u = blockIdx.x;
    const int h = static_cast<int>(u % H);
    const int jl = threadIdx.x % kCols;
    const int ig = threadIdx.x / kCols;
    const int j = blockIdx.y * kCols + jl;
    for (int x = threadIdx.x; x < d; x += kCols * kRowGroups) {
        ks[x] = load_elem(k, u * d + x);
        qs[x] = load_elem(q, u * d + x);
    }
    __syncthreads();

    float* Wu = W + u * d * d;
    const int rows = d / kRowGroups;  // 1, 2, 4 or 8
    float w[8];
    float pk = 0.f, pq = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        if (r < rows) {
            const int i = ig + kRowGroups * r;
            w[r] = Wu[i * d + j];
            pk += ks[i] * w[r];
            pq += qs[i] * w[r];
        }
    }
    red_k[ig][jl] = pk;
    red_q[ig][jl] = pq;
    if (threadIdx.x == 0) {
        float acc = 0.f;
        for (int i = 0; i < d; ++i)
            acc += qs[i] * ks[i];
        qk_s = acc;
    }
    __syncthreads();
    const float et = eta[h];
    if (ig == 0) {
        float kw = 0.f, qw = 0.f;
        for (int g = 0; g < kRowGroups; ++g) {
            kw += red_k[g][jl];
            qw += red_q[g][jl];
        }
        const float r = kw - load_elem(v, u * d + j);
        rcol[jl] = r;
        store_elem(y, u * d + j, qw - et * qk_s * r);
    }
    __syncthreads();
    const float r = rcol[jl];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        if (rr < rows) {
            const int i = ig + kRowGroups * rr;
            Wu[i * d + j] = w[rr] - et * (ks[i] * r);
        }
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a)
{
    const dim3 grid(static_cast<unsigned>(a.B * a.H), static_cast<unsigned>(a.d / kCols));
    const dim3 block(kCols * kRowGroups);
    if (a.dtype == 0)
        hipLaunchKernelGGL(decode_kernel<float>, grid, block, 0, a.stream,
                           static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                           static_cast<const float*>(a.v), a.W, a.eta, static_cast<int>(a.H),
                           a.d, static_cast<float*>(a.y));
    else
        hipLaunchKernelGGL(decode_kernel<uint16_t>, grid, block, 0, a.stream,
                           static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                           static_cast<const uint16_t*>(a.v), a.W, a.eta, static_cast<int>(a.H),
                           a.d, static_cast<uint16_t*>(a.y));
    return hipGetLastError();
}

}  // namespace ttt
