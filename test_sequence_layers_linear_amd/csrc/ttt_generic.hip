// ttt_generic.hip -- plain fp32 kernels for every shape the ABI accepts.
//
// One workgroup of 256 threads per (batch, head) chain.  Each chunk of b
// tokens runs the dual form of mini-batch gradient descent
// ("Test-Time Training Layers: How Inner-Loop Gradient Descent Replaces the
// Transformer KV Cache ...", section "Hardware Parallelization: The Dual Form
// and Mini-Batch GPU Acceleration"):
//     E = K W - V;  Y = Q W - eta tril(Q K^T) E;  W <- W - eta K^T E
// in fp32 with the tiles staged through LDS.  These kernels favour coverage
// (d in {16,32,64,128}, b in [1,64], fp32 or bf16 inputs) over speed; the
// d = 64, b = 16 bf16 shapes have dedicated MFMA kernels.
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

// ---------------------------------------------------------------------------
// TTT-Linear
// LDS: W [d][d] | Qs [b][d] | Ks [b][d] | Es [b][d] (V, then E) | S [b][b]
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ void __launch_bounds__(kThreads)
linear_generic_kernel(const TIn* __restrict__ Q, const TIn* __restrict__ K,
                      const TIn* __restrict__ V, const float* W0,
                      int w0_per_batch, const float* __restrict__ eta, int H,
                      int64_t T, int d, int b, TIn* __restrict__ Y,
                      float* W_out)
{
    extern __shared__ float lds[];
    float* Ws = lds;
    float* Qs = Ws + d * d;
    float* Ks = Qs + b * d;
    float* Es = Ks + b * d;
    float* S = Es + b * d;

    const int64_t u = blockIdx.x;
    const int h = static_cast<int>(u % H);
    const float* w0 = W0 + (w0_per_batch ? u : h) * d * d;
    for (int x = threadIdx.x; x < d * d; x += kThreads)
        Ws[x] = w0[x];
    const float et = eta[h];
    const int64_t base = u * T * d;

    for (int64_t s = 0; s < T; s += b) {
        const int n = static_cast<int>(T - s < b ? T - s : b);
        const int64_t off = base + s * d;
        __syncthreads();  // previous chunk's W update and reads are done
        load_rows(Qs, Q + off, n, d);
        load_rows(Ks, K + off, n, d);
        load_rows(Es, V + off, n, d);
        __syncthreads();
        // E = K W - V  (gradient residual at the chunk-start W)
        for (int x = threadIdx.x; x < n * d; x += kThreads) {
            const int t = x / d, j = x - t * d;
            float acc = 0.f;
            for (int i = 0; i < d; ++i)
                acc += Ks[t * d + i] * Ws[i * d + j];
            Es[x] = acc - Es[x];
        }
        // S = tril(Q K^T), diagonal included
        for (int x = threadIdx.x; x < n * n; x += kThreads) {
            const int t = x / n, t2 = x - t * n;
            float acc = 0.f;
            if (t2 <= t)
                for (int i = 0; i < d; ++i)
                    acc += Qs[t * d + i] * Ks[t2 * d + i];
            S[t * b + t2] = acc;
        }
        __syncthreads();
        // Y = Q W - eta S E
        for (int x = threadIdx.x; x < n * d; x += kThreads) {
            const int t = x / d, j = x - t * d;
            float qw = 0.f, se = 0.f;
            for (int i = 0; i < d; ++i)
                qw += Qs[t * d + i] * Ws[i * d + j];
            for (int t2 = 0; t2 <= t; ++t2)
                se += S[t * b + t2] * Es[t2 * d + j];
            store_elem(Y, off + x, qw - et * se);
        }
        __syncthreads();  // every read of W for this chunk is done
        // W <- W - eta K^T E
        for (int x = threadIdx.x; x < d * d; x += kThreads) {
            const int i = x / d, j = x - i * d;
            float acc = 0.f;
            for (int t = 0; t < n; ++t)
                acc += Ks[t * d + i] * Es[t * d + j];
            Ws[x] -= et * acc;
        }
    }
    __syncthreads();
    float* wo = W_out + u * d * d;
    for (int x = threadIdx.x; x < d * d; x += kThreads)
        wo[x] = Ws[x];
}

// ---------------------------------------------------------------------------
// TTT-MLP: the fast weights live in W1_out / W2_out (global, L2-resident per
// chain), initialised from W1_0 / W2_0 and updated in place each chunk.
// LDS: Qs, Ks, Es [b][d] | Hk, Ak, Dl, Aq [b][m] | S, Sa [b][b]
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + __expf(-x)); }

template <typename TIn>
__global__ void __launch_bounds__(kThreads)
mlp_generic_kernel(const TIn* __restrict__ Q, const TIn* __restrict__ K,
                   const TIn* __restrict__ V, const float* W1_0, const float* W2_0,
                   int w0_per_batch, const float* __restrict__ eta, int H, int64_t T,
                   int d, int m, int b, TIn* __restrict__ Y, float* W1_out, float* W2_out)
{
    extern __shared__ float lds[];
    float* Qs = lds;
    float* Ks = Qs + b * d;
    float* Es = Ks + b * d;
    float* Hk = Es + b * d;
    float* Ak = Hk + b * m;
    float* Dl = Ak + b * m;
    float* Aq = Dl + b * m;
    float* S = Aq + b * m;
    float* Sa = S + b * b;

    const int64_t u = blockIdx.x;
    const int h = static_cast<int>(u % H);
    const int64_t src = w0_per_batch ? u : h;
    const int64_t dm = static_cast<int64_t>(d) * m;
    float* W1 = W1_out + u * dm;
    float* W2 = W2_out + u * dm;
    if (W1 != W1_0 + src * dm)
        for (int x = threadIdx.x; x < dm; x += kThreads)
            W1[x] = W1_0[src * dm + x];
    if (W2 != W2_0 + src * dm)
        for (int x = threadIdx.x; x < dm; x += kThreads)
            W2[x] = W2_0[src * dm + x];
    const float et = eta[h];
    const int64_t base = u * T * d;

    for (int64_t s = 0; s < T; s += b) {
        const int n = static_cast<int>(T - s < b ? T - s : b);
        const int64_t off = base + s * d;
        __syncthreads();  // previous chunk (and the state copy) complete
        load_rows(Qs, Q + off, n, d);
        load_rows(Ks, K + off, n, d);
        load_rows(Es, V + off, n, d);
        __syncthreads();
        // Hk = K W1, Ak = SiLU(Hk);  S = tril(Q K^T)
        for (int x = threadIdx.x; x < n * m; x += kThreads) {
            const int t = x / m, p = x - t * m;
            float acc = 0.f;
            for (int i = 0; i < d; ++i)
                acc += Ks[t * d + i] * W1[i * m + p];
            Hk[x] = acc;
            Ak[x] = acc * sigmoid_f(acc);
        }
        for (int x = threadIdx.x; x < n * n; x += kThreads) {
            const int t = x / n, t2 = x - t * n;
            float acc = 0.f;
            if (t2 <= t)
                for (int i = 0; i < d; ++i)
                    acc += Qs[t * d + i] * Ks[t2 * d + i];
            S[t * b + t2] = acc;
        }
        __syncthreads();
        // E = Ak W2 - V
        for (int x = threadIdx.x; x < n * d; x += kThreads) {
            const int t = x / d, j = x - t * d;
            float acc = 0.f;
            for (int p = 0; p < m; ++p)
                acc += Ak[t * m + p] * W2[p * d + j];
            Es[x] = acc - Es[x];
        }
        __syncthreads();
        // D = (E W2^T) * SiLU'(Hk)
        for (int x = threadIdx.x; x < n * m; x += kThreads) {
            const int t = x / m, p = x - t * m;
            float acc = 0.f;
            for (int j = 0; j < d; ++j)
                acc += Es[t * d + j] * W2[p * d + j];
            const float hk = Hk[x];
            const float sg = sigmoid_f(hk);
            Dl[x] = acc * (sg * (1.0f + hk * (1.0f - sg)));
        }
        __syncthreads();
        // Hq = Q W1 - eta S D, Aq = SiLU(Hq)
        for (int x = threadIdx.x; x < n * m; x += kThreads) {
            const int t = x / m, p = x - t * m;
            float qw = 0.f, sd = 0.f;
            for (int i = 0; i < d; ++i)
                qw += Qs[t * d + i] * W1[i * m + p];
            for (int t2 = 0; t2 <= t; ++t2)
                sd += S[t * b + t2] * Dl[t2 * m + p];
            const float hq = qw - et * sd;
            Aq[x] = hq * sigmoid_f(hq);
        }
        __syncthreads();
        // Sa = tril(Aq Ak^T)
        for (int x = threadIdx.x; x < n * n; x += kThreads) {
            const int t = x / n, t2 = x - t * n;
            float acc = 0.f;
            if (t2 <= t)
                for (int p = 0; p < m; ++p)
                    acc += Aq[t * m + p] * Ak[t2 * m + p];
            Sa[t * b + t2] = acc;
        }
        __syncthreads();
        // Y = Aq W2 - eta Sa E
        for (int x = threadIdx.x; x < n * d; x += kThreads) {
            const int t = x / d, j = x - t * d;
            float aw = 0.f, se = 0.f;
            for (int p = 0; p < m; ++p)
                aw += Aq[t * m + p] * W2[p * d + j];
            for (int t2 = 0; t2 <= t; ++t2)
                se += Sa[t * b + t2] * Es[t2 * d + j];
            store_elem(Y, off + x, aw - et * se);
        }
        __syncthreads();  // every read of W1, W2 for this chunk is done
        // W1 -= eta K^T D ; W2 -= eta Ak^T E
        for (int x = threadIdx.x; x < dm; x += kThreads) {
            const int i = x / m, p = x - i * m;
            float acc = 0.f;
            for (int t = 0; t < n; ++t)
                acc += Ks[t * d + i] * Dl[t * m + p];
            W1[x] -= et * acc;
        }
        for (int x = threadIdx.x; x < dm; x += kThreads) {
            const int p = x / d, j = x - p * d;
            float acc = 0.f;
            for (int t = 0; t < n; ++t)
                acc += Ak[t * m + p] * Es[t * d + j];
            W2[x] -= et * acc;
        }
    }
}

}  // namespace

size_t linear_generic_lds_bytes(int d, int b)
{
    return sizeof(float) * (static_cast<size_t>(d) * d + 3ull * b * d + static_cast<size_t>(b) * b);
}

size_t mlp_generic_lds_bytes(int d, int m, int b)
{
    return sizeof(float) * (3ull * b * d + 4ull * b * m + 2ull * b * b);
}

template <typename Kern>
static hipError_t allow_lds(Kern kern, size_t bytes)
{
    if (bytes <= 64 * 1024)
        return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(bytes));
}

hipError_t launch_linear_generic(const LinearArgs& a)
{
    const size_t lds = linear_generic_lds_bytes(a.d, a.b);
    const dim3 grid(static_cast<unsigned>(a.B * a.H)), block(kThreads);
    if (a.dtype == 0) {
        auto kern = linear_generic_kernel<float>;
        hipError_t e = allow_lds(kern, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, grid, block, lds, a.stream,
                           static_cast<const float*>(a.Q), static_cast<const float*>(a.K),
                           static_cast<const float*>(a.V), a.W0, a.w0_per_batch, a.eta,
                           static_cast<int>(a.H), a.T, a.d, a.b, static_cast<float*>(a.Y), a.W_out);
    } else {
        auto kern = linear_generic_kernel<uint16_t>;
        hipError_t e = allow_lds(kern, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, grid, block, lds, a.stream,
                           static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                           static_cast<const uint16_t*>(a.V), a.W0, a.w0_per_batch, a.eta,
                           static_cast<int>(a.H), a.T, a.d, a.b, static_cast<uint16_t*>(a.Y),
                           a.W_out);
    }
    return hipGetLastError();
}

hipError_t launch_mlp_generic(const MlpArgs& a)
{
    const size_t lds = mlp_generic_lds_bytes(a.d, a.m, a.b);
    const dim3 grid(static_cast<unsigned>(a.B * a.H)), block(kThreads);
    if (a.dtype == 0) {
        auto kern = mlp_generic_kernel<float>;
        hipError_t e = allow_lds(kern, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, grid, block, lds, a.stream,
                           static_cast<const float*>(a.Q), static_cast<const float*>(a.K),
                           static_cast<const float*>(a.V), a.W1_0, a.W2_0, a.w0_per_batch, a.eta,
                           static_cast<int>(a.H), a.T, a.d, a.m, a.b, static_cast<float*>(a.Y),
                           a.W1_out, a.W2_out);
    } else {
        auto kern = mlp_generic_kernel<uint16_t>;
        hipError_t e = allow_lds(kern, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, grid, block, lds, a.stream,
                           static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                           static_cast<const uint16_t*>(a.V), a.W1_0, a.W2_0, a.w0_per_batch,
                           a.eta, static_cast<int>(a.H), a.T, a.d, a.m, a.b,
                           static_cast<uint16_t*>(a.Y), a.W1_out, a.W2_out);
    }
    return hipGetLastError();
}

}  // namespace ttt
