// ttt_roofs.hip -- the plain kernels behind include/ttt_roofs.h: a streaming
// copy (achievable HBM bandwidth), a dense MFMA loop (achievable matrix-core
// throughput) and an empty kernel (the cost of one launch), so that the TTT
// kernels' roofline fractions can be stated against this GPU's measured roofs
// as well as the datasheet peaks.
#include "ttt.h"
#include "ttt_roofs.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Grid-stride copy of n 16-byte elements, four loads in flight per thread,
// non-temporal loads and stores (the data is touched once).  Measured on
// MI355X for 1 GiB: 5.2 TB/s with 32 workgroups per CU, against 4.2-4.5 TB/s
// with temporal accesses, 8 loads in flight or 4-16 workgroups per CU.
__global__ void __launch_bounds__(256) roof_copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

constexpr int kChains = 8;

// kBf16: 8 independent chains of v_mfma_f32_16x16x32_bf16 per wave; else of
// v_mfma_f32_16x16x4_f32.  Operands are lane-dependent small values (the
// products must not be foldable); every thread writes the sum of its
// accumulators.
template <bool kBf16>
__global__ void __launch_bounds__(256) roof_mfma_kernel(float* __restrict__ out, int64_t iters)
{
    const int lane = threadIdx.x & 63;
    f32x4 acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j)
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kBf16) {
        bf16x8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = static_cast<__bf16>(1e-3f * static_cast<float>((lane + e) & 7));
            b[e] = static_cast<__bf16>(1e-3f * static_cast<float>((lane * 3 + e) & 7));
        }
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kChains; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
        }
    } else {
        const float a = 1e-3f * static_cast<float>(lane & 7);
        const float b = 1e-3f * static_cast<float>((lane * 3) & 7);
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kChains; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[j], 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
        s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

// No work: a launch of it costs only the dispatch and completion of its
// workgroups.
__global__ void __launch_bounds__(64) roof_launch_kernel() {}

}  // namespace

extern "C" {

int ttt_roof_copy(const void* src, void* dst, int64_t bytes, void* stream)
{
    if (!src || !dst || bytes < 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 ||
        reinterpret_cast<uintptr_t>(dst) % 16)
        return TTT_ERR_INVALID_ARG;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    if (bytes > 0 && s0 < d0 + static_cast<uintptr_t>(bytes) && d0 < s0 + static_cast<uintptr_t>(bytes))
        return TTT_ERR_INVALID_ARG;
    if (bytes == 0) return TTT_OK;
    const int64_t n = bytes / 16;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 256 * 32) blocks = 256 * 32;      // 32 workgroups per CU of a 256-CU GPU
    hipLaunchKernelGGL(roof_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       static_cast<u32x4*>(dst), n);
    return hipGetLastError() == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

int ttt_roof_mfma(float* out, int dtype, int64_t waves, int64_t iters, double* flops, void* stream)
{
    if (!out || (dtype != TTT_F32 && dtype != TTT_BF16) || waves < 4 || waves % 4 != 0 ||
        waves / 4 > 0x7fffffff || iters < 1)
        return TTT_ERR_INVALID_ARG;
    const double per = dtype == TTT_BF16 ? 2.0 * 16 * 16 * 32 : 2.0 * 16 * 16 * 4;
    if (flops) *flops = static_cast<double>(waves) * static_cast<double>(iters) * kChains * per;
    const dim3 grid(static_cast<unsigned>(waves / 4)), block(256);
    if (dtype == TTT_BF16)
        hipLaunchKernelGGL(roof_mfma_kernel<true>, grid, block, 0, static_cast<hipStream_t>(stream),
                           out, iters);
    else
        hipLaunchKernelGGL(roof_mfma_kernel<false>, grid, block, 0, static_cast<hipStream_t>(stream),
                           out, iters);
    return hipGetLastError() == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

int ttt_roof_launch(int64_t workgroups, void* stream)
{
    if (workgroups < 1 || workgroups > 0x7fffffff)
        return TTT_ERR_INVALID_ARG;
    hipLaunchKernelGGL(roof_launch_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(64), 0,
                       static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

}  // extern "C"
