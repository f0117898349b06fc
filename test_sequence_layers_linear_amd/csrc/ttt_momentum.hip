// ttt_momentum.hip -- TTT-Linear with momentum gradient descent (the E2-TTT
// write-up on zhichai.net, sections "E2-TTT's Breakthrough: A Closed-Form
// Solution" and "Core Math (Simplified)"): fast weights W and a momentum M,
// one step per token on the squared loss 1/2 ||k W - v||^2,
//     M_t = beta M_{t-1} + k_t^T r_t,   W_t = W_{t-1} - eta M_t,   y_t = q_t W_t,
// with the residual r_t = k_t W_g - v_t taken at W_g = W_{t-1} (grad_mode 0:
// exact token-level steps) or at the chunk-start weights (grad_mode 1: the
// chunk-start gradients of the section "The Curse of Efficiency").
//
// Chunk closed form (derived here; the page states that one exists but its
// formula is missing).  For a chunk of n tokens starting from (W, M), token t
// (0-based) sees the weights after the chunk's first t tokens,
//     W_(t) = W - eta c_t M - eta sum_{u<t} dsum_{t-1-u} k_u^T r_u,
//     c_t = beta + ... + beta^t,   dsum_m = 1 + beta + ... + beta^m,
// so with E = K W - V:
//   grad_mode 0: (I + eta A) R = E - eta diag(c_t) K M,
//                A[t][u] = dsum_{t-1-u} (k_t . k_u) for u < t, else 0,
//                a unit lower triangular system (one forward substitution);
//   grad_mode 1: R = E;
// and then
//   Y      = Q W - eta diag(c_{t+1}) Q M - eta (S o Dsum) R,
//            S = tril(Q K^T) (diagonal kept), Dsum[t][u] = dsum_{t-u}
//   W_next = W - eta c_n M - eta K^T diag(dsum_{n-1-u}) R
//   M_next = beta^n M + K^T diag(beta^{n-1-u}) R.
// With beta = 0: c = 0, dsum = 1, and grad_mode 1 is the mini-batch dual
// form, grad_mode 0 exact online gradient descent (the delta rule).
//
// This file holds the plain fp32 kernel for every shape the ABI accepts:
// one workgroup of 256 threads per (batch, head) chain, W and M in LDS.
#include "ttt_internal.h"

namespace ttt {
namespace {

constexpr int kThreads = 256;

template <typename TIn>
__device__ void load_rows(float* dst, const TIn* src, int n, int d)
{
    for (int x = threadIdx.x; x < n * d; x += kThreads)
        dst[x] = load_elem(src, x);
}

// LDS: W, M [d][d] | Qs, Ks, Rs [b][d] (Rs: V, then the residuals) |
//      G, S [b][b] | pw, cs, ds [b + 1]
template <typename TIn>
__global__ void __launch_bounds__(kThreads)
momentum_generic_kernel(const TIn* __restrict__ Q, const TIn* __restrict__ K,
                        const TIn* __restrict__ V, const float* W0, int w0_per_batch,
                        const float* M0, const float* __restrict__ eta,
                        const float* __restrict__ beta, int grad_mode, int H, int64_t T,
                        int d, int b, TIn* __restrict__ Y, float* W_out, float* M_out)
{
    extern __shared__ float lds[];
    float* Ws = lds;
    float* Ms = Ws + d * d;
    float* Qs = Ms + d * d;
    float* Ks = Qs + b * d;
    float* Rs = Ks + b * d;
    float* G = Rs + b * d;
    float* S = G + b * b;
    float* pw = S + b * b;      // beta^m
    float* cs = pw + b + 1;     // c_t = beta + ... + beta^t (c_0 = 0)
    float* ds = cs + b + 1;     // dsum_m = 1 + beta + ... + beta^m

    const int64_t u = blockIdx.x;
    const int h = static_cast<int>(u % H);
    const float* w0 = W0 + (w0_per_batch ? u : h) * d * d;
    for (int x = threadIdx.x; x < d * d; x += kThreads) {
        Ws[x] = w0[x];
        Ms[x] = M0 ? M0[u * d * d + x] : 0.f;
    }
    const float et = eta[h], bt = beta[h];
    if (threadIdx.x == 0) {
        float p = 1.f;
        pw[0] = 1.f;
        cs[0] = 0.f;
        ds[0] = 1.f;
        for (int m = 1; m <= b; ++m) {
            p *= bt;
            pw[m] = p;
            cs[m] = cs[m - 1] + p;
            ds[m] = ds[m - 1] + p;
        }
    }
    const bool exact = grad_mode == 0;
    const int64_t base = u * T * d;

    for (int64_t s = 0; s < T; s += b) {
        const int n = static_cast<int>(T - s < b ? T - s : b);
        const int64_t off = base + s * d;
        __syncthreads();  // previous chunk's state update (and the set-up) done
        load_rows(Qs, Q + off, n, d);
        load_rows(Ks, K + off, n, d);
        load_rows(Rs, V + off, n, d);
        __syncthreads();
        // right-hand side: k_t W - v_t (- eta c_t k_t M for exact steps)
        for (int x = threadIdx.x; x < n * d; x += kThreads) {
            const int t = x / d, j = x - t * d;
            float kw = 0.f, km = 0.f;
            for (int i = 0; i < d; ++i) {
                kw += Ks[t * d + i] * Ws[i * d + j];
                km += Ks[t * d + i] * Ms[i * d + j];
            }
            Rs[x] = kw - Rs[x] - (exact ? et * cs[t] * km : 0.f);
        }
        // G = eta A (exact steps), S = eta (tril(Q K^T) o Dsum)
        for (int x = threadIdx.x; x < n * n; x += kThreads) {
            const int t = x / n, t2 = x - t * n;
            float kk = 0.f, qk = 0.f;
            for (int i = 0; i < d; ++i) {
                kk += Ks[t * d + i] * Ks[t2 * d + i];
                qk += Qs[t * d + i] * Ks[t2 * d + i];
            }
            G[t * b + t2] = (exact && t2 < t) ? et * ds[t - 1 - t2] * kk : 0.f;
            S[t * b + t2] = t2 <= t ? et * ds[t - t2] * qk : 0.f;
        }
        __syncthreads();
        // exact steps: forward substitution, one column per thread
        if (exact) {
            for (int j = threadIdx.x; j < d; j += kThreads)
                for (int t = 1; t < n; ++t) {
                    float acc = Rs[t * d + j];
                    for (int t2 = 0; t2 < t; ++t2)
                        acc -= G[t * b + t2] * Rs[t2 * d + j];
                    Rs[t * d + j] = acc;
                }
            __syncthreads();
        }
        // Y = Q W - eta diag(c_{t+1}) Q M - S R
        for (int x = threadIdx.x; x < n * d; x += kThreads) {
            const int t = x / d, j = x - t * d;
            const float cq = et * cs[t + 1];
            float qw = 0.f, sr = 0.f;
            for (int i = 0; i < d; ++i)
                qw += Qs[t * d + i] * (Ws[i * d + j] - cq * Ms[i * d + j]);
            for (int t2 = 0; t2 <= t; ++t2)
                sr += S[t * b + t2] * Rs[t2 * d + j];
            store_elem(Y, off + x, qw - sr);
        }
        __syncthreads();  // every read of W and M for this chunk is done
        // W -= eta c_n M + eta K^T diag(dsum) R;  M = beta^n M + K^T diag(beta^.) R
        const float cw = et * cs[n], cm = pw[n];
        for (int x = threadIdx.x; x < d * d; x += kThreads) {
            const int i = x / d, j = x - i * d;
            float aw = 0.f, am = 0.f;
            for (int t = 0; t < n; ++t) {
                const float kr = Ks[t * d + i] * Rs[t * d + j];
                aw += ds[n - 1 - t] * kr;
                am += pw[n - 1 - t] * kr;
            }
            const float m = Ms[x];
            Ws[x] = Ws[x] - cw * m - et * aw;
            Ms[x] = cm * m + am;
        }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < d * d; x += kThreads) {
        W_out[u * d * d + x] = Ws[x];
        M_out[u * d * d + x] = Ms[x];
    }
}

template <typename Kern>
hipError_t allow_lds(Kern kern, size_t bytes)
{
    if (bytes <= 64 * 1024)
        return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(bytes));
}

template <typename TIn>
hipError_t launch_generic_t(const MomentumArgs& a)
{
    const size_t lds = momentum_generic_lds_bytes(a.d, a.b);
    auto kern = momentum_generic_kernel<TIn>;
    hipError_t e = allow_lds(kern, lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(a.B * a.H)), dim3(kThreads), lds,
                       a.stream, static_cast<const TIn*>(a.Q), static_cast<const TIn*>(a.K),
                       static_cast<const TIn*>(a.V), a.W0, a.w0_per_batch, a.M0, a.eta, a.beta,
                       a.grad_mode, static_cast<int>(a.H), a.T, a.d, a.b,
                       static_cast<TIn*>(a.Y), a.W_out, a.M_out);
    return hipGetLastError();
}

}  // namespace

size_t momentum_generic_lds_bytes(int d, int b)
{
    return sizeof(float) * (2ull * d * d + 3ull * b * d + 2ull * b * b + 3ull * (b + 1));
}

hipError_t launch_momentum_generic(const MomentumArgs& a)
{
    return a.dtype == 0 ? launch_generic_t<float>(a) : launch_generic_t<uint16_t>(a);
}

}  // namespace ttt
