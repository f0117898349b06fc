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
// the updated column, so W is read once and written once.  Every global load
// is issued before the first barrier (one trip to memory per step), and
// q . k is summed like k W_j and q W_j, from per-thread partials.
//
// kPro: the input prologue of ttt_linear_forward_ex for one token: q and k
// LayerNorm'd over the head dim (waves 0 and 1, one row each, butterfly sums
// over the wave), the token's own step size, and with read_start the readout
// before the update (y = q W), the b = 1 case of the chunk-start read.
#include "ttt_internal.h"

namespace ttt {
namespace {

constexpr int kCols = 16;
constexpr int kRowGroups = 16;

// LayerNorm of the d <= 128 values in buf (LDS) by one whole wave: lane l
// holds elements l and l + 64
__device__ void layernorm_wave(float* buf, int d, const float* __restrict__ prm, int h, float eps)
{
    const int l = threadIdx.x & 63;
    const float x0 = l < d ? buf[l] : 0.f;
    const float x1 = l + 64 < d ? buf[l + 64] : 0.f;
    float sum = x0 + x1;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        sum += __shfl_xor(sum, m);
    const float mean = sum / static_cast<float>(d);
    const float d0 = l < d ? x0 - mean : 0.f;
    const float d1 = l + 64 < d ? x1 - mean : 0.f;
    float sq = d0 * d0 + d1 * d1;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        sq += __shfl_xor(sq, m);
    const float rstd = rsqrtf(sq / static_cast<float>(d) + eps);
    if (l < d)
        buf[l] = d0 * rstd * prm[(2 * h) * d + l] + prm[(2 * h + 1) * d + l];
    if (l + 64 < d)
        buf[l + 64] = d1 * rstd * prm[(2 * h) * d + l + 64] + prm[(2 * h + 1) * d + l + 64];
}

template <typename TIn, bool kPro>
__global__ void __launch_bounds__(kCols * kRowGroups)
decode_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
              const TIn* __restrict__ v, float* __restrict__ W,
              const float* __restrict__ eta, int H, int d, TIn* __restrict__ y, Prologue pro)
{
    __shared__ float ks[128], qs[128];
    __shared__ float red_k[kRowGroups][kCols + 1], red_q[kRowGroups][kCols + 1];
    __shared__ float red_qk[kRowGroups];
    __shared__ float rcol[kCols];

    const int64_t u = blockIdx.x;
    const int h = static_cast<int>(u % H);
    const int jl = threadIdx.x % kCols;
    const int ig = threadIdx.x / kCols;
    const int j = blockIdx.y * kCols + jl;
    const int rows = d / kRowGroups;  // 1, 2, 4 or 8

    // every global load first, so the step costs one trip to memory: this
    // thread's d / 16 rows of column j of W, v_j, and (plain step) the k and
    // q entries of those rows
    float* Wu = W + u * d * d;
    float w[8], kr[8], qr[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
        if (r < rows)
            w[r] = Wu[(ig + kRowGroups * r) * d + j];
    const float vj = load_elem(v, u * d + j);
    const float et = (kPro && pro.eta_tok) ? pro.eta_tok[u] : eta[h];
    if constexpr (kPro) {
        // the LayerNorm needs whole rows: stage k and q in LDS
        for (int x = threadIdx.x; x < d; x += kCols * kRowGroups) {
            ks[x] = load_elem(k, u * d + x);
            qs[x] = load_elem(q, u * d + x);
        }
        __syncthreads();
        if (pro.ln_k || pro.ln_q) {
            const int wv = threadIdx.x >> 6;          // wave-uniform roles
            if (wv == 0 && pro.ln_k)
                layernorm_wave(ks, d, pro.ln_k, h, pro.ln_eps);
            if (wv == 1 && pro.ln_q)
                layernorm_wave(qs, d, pro.ln_q, h, pro.ln_eps);
            __syncthreads();
        }
#pragma unroll
        for (int r = 0; r < 8; ++r)
            if (r < rows) {
                kr[r] = ks[ig + kRowGroups * r];
                qr[r] = qs[ig + kRowGroups * r];
            }
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r)
            if (r < rows) {
                kr[r] = load_elem(k, u * d + ig + kRowGroups * r);
                qr[r] = load_elem(q, u * d + ig + kRowGroups * r);
            }
    }

    // partial k W_j, q W_j and q . k over this thread's rows, then the sums
    // over the 16 row groups
    float pk = 0.f, pq = 0.f, pqk = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r)
        if (r < rows) {
            pk += kr[r] * w[r];
            pq += qr[r] * w[r];
            pqk += qr[r] * kr[r];
        }
    red_k[ig][jl] = pk;
    red_q[ig][jl] = pq;
    if (jl == 0)
        red_qk[ig] = pqk;
    __syncthreads();
    if (ig == 0) {
        float kw = 0.f, qw = 0.f, qk = 0.f;
        for (int g = 0; g < kRowGroups; ++g) {
            kw += red_k[g][jl];
            qw += red_q[g][jl];
            qk += red_qk[g];
        }
        const float r = kw - vj;
        rcol[jl] = r;
        store_elem(y, u * d + j, (kPro && pro.read_start) ? qw : qw - et * qk * r);
    }
    __syncthreads();
    const float r = rcol[jl];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr)
        if (rr < rows)
            Wu[(ig + kRowGroups * rr) * d + j] = w[rr] - et * (kr[rr] * r);
}

template <bool kPro>
hipError_t launch(const DecodeArgs& a)
{
    const dim3 grid(static_cast<unsigned>(a.B * a.H), static_cast<unsigned>(a.d / kCols));
    const dim3 block(kCols * kRowGroups);
    if (a.dtype == 0)
        hipLaunchKernelGGL((decode_kernel<float, kPro>), grid, block, 0, a.stream,
                           static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                           static_cast<const float*>(a.v), a.W, a.eta, static_cast<int>(a.H),
                           a.d, static_cast<float*>(a.y), a.pro);
    else
        hipLaunchKernelGGL((decode_kernel<uint16_t, kPro>), grid, block, 0, a.stream,
                           static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                           static_cast<const uint16_t*>(a.v), a.W, a.eta, static_cast<int>(a.H),
                           a.d, static_cast<uint16_t*>(a.y), a.pro);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a)
{
    return a.pro.active() ? launch<true>(a) : launch<false>(a);
}

}  // namespace ttt
