// ttt_decode.hip -- single-token TTT-Linear step (online gradient descent):
//     r = k W - v;   W <- W - eta k^T r;   y = q W (updated)
// ("Test-Time Training Layers: How Inner-Loop Gradient Descent Replaces the
// Transformer KV Cache ...", section "The Core Mechanism", steps 1-3; its
// section "Hardware Parallelization" names this sequential form as the one
// for token-by-token decoding with O(1) step cost).
//
// The step is bound by the fp32 state (read + write d*d*4 bytes per
// (batch, head)) and, at these sizes, by latency: one trip to memory and
// back plus the launch.  Output columns of W are independent (column j needs
// only W[:, j], k, q and v_j), so one wave serves 32 columns of one
// (batch, head) with 16-byte accesses and no LDS or barrier.  y_j uses
// q W'_j = q W_j - eta (q . k) r_j, algebraically the readout with the
// updated column, so W is read once and written once, and every global load
// is issued before any arithmetic.
//
// kPro: the input prologue of ttt_linear_forward_ex for one token: q and k
// LayerNorm'd over the head dim, the token's own step size, and with
// read_start the readout before the update (y = q W), the b = 1 case of the
// chunk-start read.
#include "ttt_internal.h"

namespace ttt {
namespace {

// Column groups of 4 per wave: 8, i.e. 32 columns per wave and two waves per
// (batch, head) at d = 64.  Measured on MI355X for 48 heads in a HIP graph of
// 256 steps: 2.07 us per step, against 2.36 with 64 columns per wave (one
// wave per head: twice the loads per lane in one wave) and 2.48 with 16.
// The other 3 lane bits number the row groups, so that every sum over the
// input index ends inside an aligned octet of lanes.
constexpr int kDecodeColumnGroups = 8;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// R consecutive q/k elements of the lane's row block (fp32 or bf16) in fp32,
// in the widest loads the block allows (16 bytes where it can).
template <int R>
__device__ __forceinline__ void load_block(const float* p, float (&x)[R])
{
    if constexpr (R % 4 == 0) {
#pragma unroll
        for (int i = 0; i < R; i += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(p + i);
            x[i] = v[0]; x[i + 1] = v[1]; x[i + 2] = v[2]; x[i + 3] = v[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < R; ++i)
            x[i] = p[i];
    }
}
template <int R>
__device__ __forceinline__ void load_block(const uint16_t* p, float (&x)[R])
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    if constexpr (R % 8 == 0) {
#pragma unroll
        for (int i = 0; i < R; i += 8) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(p + i);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[i + 2 * e] = __uint_as_float(v[e] << 16);
                x[i + 2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
            }
        }
    } else if constexpr (R == 4) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(p);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            x[2 * e] = __uint_as_float(v[e] << 16);
            x[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < R; ++i)
            x[i] = __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
    }
}

// x of the lane that DPP control `ctrl` selects, within the lane's row of 16
template <int kCtrl>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, false));
}

// Sum over the wave's 8 row groups: the lanes of an aligned octet (the row
// group is lane % 8).  Three DPP adds, no LDS round trip: swap neighbours
// (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), after which the four
// lanes of a quad hold its sum, then mirror the octet (lane i reads lane
// 7 - i, in the other quad).  Each add is commutative in its two operands,
// so every lane of the octet ends with the same bits.
__device__ __forceinline__ float rowgroup_sum(float x)
{
    x += dpp<0xb1>(x);       // quad_perm [1, 0, 3, 2]
    x += dpp<0x4e>(x);       // quad_perm [2, 3, 0, 1]
    x += dpp<0x141>(x);      // row_half_mirror
    return x;
}

// One wave per (batch, head) and slice of 4 kCG columns of W.  Lane l holds
// the four columns j = 4 kCG slice + 4 (l / 8) .. + 3 over the R rows
// (l % 8) R .. + R - 1, R = d kCG / 64: each of its R float4 loads and
// stores is one row segment.  Sums over the input index run over the lane's
// rows, then over the 8 row groups of its octet (rowgroup_sum).  k and q:
// each lane reads its R-row block.
template <typename TIn, int kD, bool kPro, int kCG>
__global__ void __launch_bounds__(64)
decode_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
              const TIn* __restrict__ v, float* __restrict__ W,
              const float* __restrict__ eta, int H, TIn* __restrict__ y, Prologue pro)
{
    constexpr int kCols = 4 * kCG;                // columns per wave
    constexpr int kSlices = (kD + kCols - 1) / kCols;
    constexpr int R = kD * kCG / 64;              // rows per lane
    constexpr int kGroups = kD / 4 < kCG ? kD / 4 : kCG;   // column groups in use
    static_assert(64 / kCG == 8, "rowgroup_sum adds the 8 row groups of a lane octet");
    const int lane = threadIdx.x;
    const int64_t u = blockIdx.x / kSlices;
    const int cg = lane >> 3, rg = lane & 7;
    // d < 32: the octets past the last column group repeat column group 0
    // and store nothing (a constant true otherwise, so that no branch gives
    // the compiler a place to sink the loads of v and eta into)
    const bool active = kGroups == kCG || cg < kGroups;
    const int j0 = (blockIdx.x % kSlices) * kCols + 4 * (active ? cg : 0);
    const int h = static_cast<int>(u % H);
    const int i0 = rg * R;

    // every global load first: one trip to memory per step
    float* Wu = W + u * kD * kD;
    f32x4 w[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        w[i] = *reinterpret_cast<const f32x4*>(Wu + (i0 + i) * kD + j0);
    float kr[R], qr[R];
    load_block<R>(k + u * kD + i0, kr);
    load_block<R>(q + u * kD + i0, qr);
    float vj[4];
    load_block<4>(v + u * kD + j0, vj);
    const float et = (kPro && pro.eta_tok) ? pro.eta_tok[u] : eta[h];
    // (all of them in flight before the first use: left to itself the
    // scheduler issues the last W row only after the first rows arrive)
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (kPro) {
        // LayerNorm of the whole k and q rows: each row group holds R of the
        // d elements; the sums run over the lane's block, then the groups
        auto norm = [&](float (&x)[R], const float* prm) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < R; ++i)
                s += x[i];
            const float mean = rowgroup_sum(s) * (1.0f / kD);
            float sq = 0.f;
#pragma unroll
            for (int i = 0; i < R; ++i)
                sq += (x[i] - mean) * (x[i] - mean);
            const float rstd = rsqrtf(rowgroup_sum(sq) * (1.0f / kD) + pro.ln_eps);
#pragma unroll
            for (int i = 0; i < R; ++i)
                x[i] = (x[i] - mean) * rstd * prm[(2 * h) * kD + i0 + i] + prm[(2 * h + 1) * kD + i0 + i];
        };
        if (pro.ln_k)
            norm(kr, pro.ln_k);
        if (pro.ln_q)
            norm(qr, pro.ln_q);
    }

    // k W_j, q W_j over the lane's rows, and q . k, then over the row groups
    float kw[4] = {0.f, 0.f, 0.f, 0.f}, qw[4] = {0.f, 0.f, 0.f, 0.f}, qk = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kw[e] += kr[i] * w[i][e];
            qw[e] += qr[i] * w[i][e];
        }
        qk += qr[i] * kr[i];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        kw[e] = rowgroup_sum(kw[e]);
        qw[e] = rowgroup_sum(qw[e]);
    }
    qk = rowgroup_sum(qk);
    if (!active)
        return;
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        r[e] = kw[e] - vj[e];
    // q W'_j = q W_j - eta (q . k) r_j: the readout with the updated column
    if (rg == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            store_elem(y, u * kD + j0 + e, (kPro && pro.read_start) ? qw[e] : qw[e] - et * qk * r[e]);
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = w[i][e] - et * (kr[i] * r[e]);
        *reinterpret_cast<f32x4*>(Wu + (i0 + i) * kD + j0) = o;
    }
}

template <typename TIn, int kD, bool kPro>
void launch_d(const DecodeArgs& a)
{
    constexpr int kCG = kDecodeColumnGroups;
    constexpr int kSlices = (kD + 4 * kCG - 1) / (4 * kCG);
    const dim3 grid(static_cast<unsigned>(a.B * a.H * kSlices));
    hipLaunchKernelGGL((decode_kernel<TIn, kD, kPro, kCG>), grid, dim3(64), 0, a.stream,
                       static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                       static_cast<const TIn*>(a.v), a.W, a.eta, static_cast<int>(a.H),
                       static_cast<TIn*>(a.y), a.pro);
}

template <typename TIn, bool kPro>
void launch_t(const DecodeArgs& a)
{
    switch (a.d) {
    case 16: launch_d<TIn, 16, kPro>(a); break;
    case 32: launch_d<TIn, 32, kPro>(a); break;
    case 64: launch_d<TIn, 64, kPro>(a); break;
    default: launch_d<TIn, 128, kPro>(a); break;
    }
}

template <bool kPro>
hipError_t launch(const DecodeArgs& a)
{
    if (a.dtype == 0)
        launch_t<float, kPro>(a);
    else
        launch_t<uint16_t, kPro>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a)
{
    return a.pro.active() ? launch<true>(a) : launch<false>(a);
}

}  // namespace ttt
