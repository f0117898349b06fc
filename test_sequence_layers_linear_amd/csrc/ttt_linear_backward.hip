// ttt_linear_backward.hip -- backward of the TTT-Linear dual-form scan for
// head dim d = 64 and mini-batch b = 16, fp32 or bf16 Q/K/V, fp32 state.
//
// Outer-loop training differentiates the layer output through the inner
// updates ("Test-Time Training Layers: How Inner-Loop Gradient Descent
// Replaces the Transformer KV Cache ...", section "Hardware Parallelization:
// The Dual Form and Mini-Batch GPU Acceleration": the dual form exists so the
// layer trains efficiently; the uTTT write-up on thelatestinai.com, Figure
// 2(b): the read-output Jacobian runs backward through the earlier inner
// updates).  Given the cotangents dY of Y and dW_out of the final state, one
// chunk of the forward
//     E = K W - V,   A = tril(Q K^T),   Y = Q W - eta A E,   W' = W - eta K^T E
// has, with G' the cotangent of W' (G' = dW_out after the last chunk),
//     P   = A^T dY + K G'           dE = -eta P     deta += -<P, E>
//     dA  = -eta tril(dY E^T)
//     dQ  = dY W^T + dA K
//     dK  = -eta (P W^T + E G'^T) + dA^T Q
//     dV  = eta P
//     G   = G' + Q^T dY + K^T dE    (the cotangent of the chunk-start W)
// and dW0 is G after the first chunk.
//
// One workgroup of 4 waves per (batch, head) chain:
//   sweep 1 (forward): recompute the chunk-start state W_c of every chunk and
//     store it in the workspace (16 KB per chunk), wave w updating the 16
//     output columns [16w, 16w + 16) of W (the loss separates over output
//     columns);
//   sweep 2 (reverse over the chunks): phase A is column-local, wave w owns
//     columns [16w, 16w + 16) of E, P, dE and of the cotangent G (kept in
//     registers); phase B needs sums over all 64 columns, so wave w there owns
//     input dims [16w, 16w + 16) of dQ, dK (and dV), reading E, P and G' that
//     phase A left in LDS.  Two barriers per chunk.
// Every product is a v_mfma_f32_16x16x4_f32 (one MFMA shape throughout).
// Layouts (lane l, c = l % 16, g = l / 16): A operand A[c][k-slot g], B
// operand B[k-slot g][c], accumulator rows 4g..4g+3 of column c.  An
// accumulator tile is therefore the B operand of a product over its row
// index (k-step r takes register r: k = 4g + r) and, read as an A operand,
// the transpose of itself -- which is how S = Q K^T turns into A^T and dA
// into dA^T without data movement.
//
// Inputs of a chunk (Q, K, dY as fp32) are staged through a two-slot LDS
// ring, the next chunk's global loads issued before this chunk's products;
// each wave loads the 16 V columns it needs straight into registers, and W_c
// has one LDS buffer: every wave reads the W rows it needs in phase B before
// the mid-chunk barrier, so the next W_c is written right after that barrier.
// That keeps a workgroup at 73 KB of LDS and under 256 VGPRs (two fit on a
// CU; measured, two per CU run at half the speed each: the chunk is bound by
// the SIMD's VALU and fp32 MFMA issue, so the segment planner keeps one per
// CU).  LDS rows are
// padded to 68 floats so the 16 rows a 16-lane group reads fall in different
// banks.  Tokens past T read as zero: they add nothing to any product, and
// their rows are not stored.
//
// kPro: the input prologue, as in the bf16 kernel (ttt_linear_backward_bf16.hip):
// Q, K LayerNorm'd while staged (the staging threads keep xh and 1/std),
// per-token step sizes (E, P, dK, dV scale by row, dA by column), the
// chunk-start read dropping A, and an epilogue in which the staging threads
// apply the LayerNorm backward to dQ, dK of the normalised rows (through LDS),
// store them and sum the gamma, beta gradients.  83 KB of LDS: one per CU.
#include "ttt_mfma_ops.h"

namespace ttt {
namespace {

constexpr int kD = 64;
constexpr int kB = 16;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kP = 68;                          // padded LDS row, floats
constexpr int kTile = kB * kP;                  // a 16 x 64 tile
constexpr int kWTile = kD * kP;                 // a 64 x 64 matrix
constexpr int kSlotQ = 0;
constexpr int kSlotK = kTile;
constexpr int kSlotDY = 2 * kTile;
constexpr int kSlotFloats = 3 * kTile;          // one chunk's Q, K, dY
constexpr int kOffW = 2 * kSlotFloats;          // W_c [64][kP], one buffer
constexpr int kOffE = kOffW + kWTile;           // E  [16][kP]
constexpr int kOffP = kOffE + kTile;            // P  [16][kP]
constexpr int kOffG = kOffP + kTile;            // G' [64][kP]
constexpr int kDAP = 20;                        // padded row of a wave's dA copy
constexpr int kOffDA = kOffG + kWTile;          // [4 waves][16][kDAP]
constexpr int kOffRed = kOffDA + kWaves * kB * kDAP;
constexpr int kLdsFloats = kOffRed + kWaves;
constexpr int kLdsBytes = kLdsFloats * 4;       // 74768
constexpr int kGMapLdsBytes = 2 * kSlotFloats * 4;   // the cotangent maps use the slots only
static_assert(2 * kLdsBytes <= kMaxLdsBytes, "two workgroups per CU");
// prologue additions (floats), after the plain layout; the cotangent maps
// put the slots' step sizes right after the slots
constexpr int kOffEtaMain = kLdsFloats;          // [2 slots][16] eta_t
constexpr int kOffEtaGMap = 2 * kSlotFloats;
constexpr int kOffDQ = kOffEtaMain + 2 * kB;     // [16][kP] dQ of the normalised rows
constexpr int kOffDK = kOffDQ + kTile;
constexpr int kOffDeta = kOffDK + kTile;         // [4 waves][16]
constexpr int kProLdsBytes = (kOffDeta + kWaves * kB) * 4;
constexpr int kProGMapLdsBytes = (kOffEtaGMap + 2 * kB) * 4;
static_assert(kProLdsBytes <= kMaxLdsBytes, "one workgroup per CU");
static_assert(kWaves * 4 * kD <= 2 * kTile, "the gamma/beta reduction fits the dQ, dK tiles");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four consecutive elements of a row as fp32 (raw register form while the
// load is in flight, converted when written to LDS).
template <typename In> struct Raw;
template <> struct Raw<float> {
    typedef f32x4 type;
    __device__ static type load(const float* p, bool ok)
    {
        return ok ? *reinterpret_cast<const f32x4*>(p) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __device__ static f32x4 to_f32(type x) { return x; }
};
template <> struct Raw<uint16_t> {
    typedef u32x2 type;
    __device__ static type load(const uint16_t* p, bool ok)
    {
        return ok ? *reinterpret_cast<const u32x2*>(p) : u32x2{0u, 0u};
    }
    __device__ static f32x4 to_f32(type x)
    {
        return f32x4{__uint_as_float(x[0] << 16), __uint_as_float(x[0] & 0xffff0000u),
                     __uint_as_float(x[1] << 16), __uint_as_float(x[1] & 0xffff0000u)};
    }
};

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

template <typename In>
struct Stage {
    typename Raw<In>::type q, k, dy;
    In v[4];           // V[4g + r][16w + c]: this lane's entries of its wave's columns
    f32x4 w[4];
    float eta;         // kPro: the step size of row tid / 16 (0 past T)
    bool ok;           // row tid / 16 is a token (< T)
};

// four consecutive outputs of a row: 16 bytes (fp32) or 8 bytes (bf16)
__device__ __forceinline__ void store_row4(float* p, const float (&x)[4])
{
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
}
__device__ __forceinline__ void store_row4(uint16_t* p, const float (&x)[4])
{
    *reinterpret_cast<u32x2*>(p) = u32x2{static_cast<uint32_t>(f32_to_bf16_bits(x[0])) |
                                             (static_cast<uint32_t>(f32_to_bf16_bits(x[1])) << 16),
                                         static_cast<uint32_t>(f32_to_bf16_bits(x[2])) |
                                             (static_cast<uint32_t>(f32_to_bf16_bits(x[3])) << 16)};
}

__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void lds4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }

// kGMap = false: the backward of segment s of a chain (all of it when
//   nseg = 1): sweep 1 recomputes the segment's chunk-start states from its
//   start state (W0, or wstart[u][s]) into the workspace, sweep 2 runs from the
//   cotangent of the segment's end state (dW_out, or gend[u][nseg - 1 - s])
//   back to its start, writing dQ, dK, dV of the segment's rows, the
//   segment's share of deta and, for segment 0, dW0 of the chain.
// kGMap = true: the affine map of the cotangent over segment s >= 1,
//   G_start = M^G G_end + N^G (M^G from G_end = I with dY = 0, block half 0;
//   N^G from G_end = 0 with the segment's dY, half 1), stored in the order
//   the composition runs: gmaps[u][nseg - 1 - s][half].  No W is needed.
template <typename In, bool kGMap, bool kPro>
__global__ void __launch_bounds__(kThreads, kPro && !kGMap ? 1 : 2)
linear_backward_kernel(const In* __restrict__ Q, const In* __restrict__ K, const In* __restrict__ V,
                       const float* __restrict__ W0, int w0_per_batch,
                       const float* __restrict__ eta, int H, int T, int64_t units, int seg_len,
                       int nseg, const float* __restrict__ wstart, const float* __restrict__ gend,
                       const In* __restrict__ dY, const float* __restrict__ dW_out,
                       In* __restrict__ dQ, In* __restrict__ dK, In* __restrict__ dV,
                       float* __restrict__ dW0_chain, float* __restrict__ deta_chain,
                       float* __restrict__ states, float* __restrict__ gmaps,
                       Prologue pro, float* __restrict__ deta_tok, float* __restrict__ dln_chain)
{
    extern __shared__ __attribute__((aligned(16))) float lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;

    int64_t u = blockIdx.x;
    int s = 0, half = 0;
    if (nseg > 1) {
        xcd_block(blockIdx.x, kGMap ? 2 * (nseg - 1) : nseg, units, u, s);
        if (u >= units)                  // padding of the XCD placement
            return;
        if (kGMap) {
            half = s & 1;
            s = (s >> 1) + 1;
        }
    }
    const int h = static_cast<int>(u % H);
    const float et = eta[h];
    const int seg_chunks = seg_len / kB;
    const int c0 = s * seg_chunks;
    const int c1 = min((T + kB - 1) / kB, c0 + seg_chunks);
    const int64_t off = u * static_cast<int64_t>(T) * kD;
    float* st = states + (u * nseg + s) * static_cast<int64_t>(seg_chunks) * kD * kD;
    static_assert(sizeof(In) == 4, "fp32 rows (bf16 inputs run in ttt_linear_backward_bf16.hip)");
    const int64_t chain_bytes = static_cast<int64_t>(T) * kD * 4;
    const __amdgpu_buffer_rsrc_t r_q = mfma::buffer_rsrc(Q + off, chain_bytes);
    const __amdgpu_buffer_rsrc_t r_k = mfma::buffer_rsrc(K + off, chain_bytes);
    const __amdgpu_buffer_rsrc_t r_v = mfma::buffer_rsrc(V + off, kGMap ? 0 : chain_bytes);
    const __amdgpu_buffer_rsrc_t r_dy = mfma::buffer_rsrc(dY + off, chain_bytes);
    const __amdgpu_buffer_rsrc_t r_dq = mfma::buffer_rsrc(dQ + off, kGMap ? 0 : chain_bytes);
    const __amdgpu_buffer_rsrc_t r_dk = mfma::buffer_rsrc(dK + off, kGMap ? 0 : chain_bytes);
    const __amdgpu_buffer_rsrc_t r_dv = mfma::buffer_rsrc(dV + off, kGMap ? 0 : chain_bytes);
    // this segment's chunk-start states in the workspace
    const __amdgpu_buffer_rsrc_t r_st =
        mfma::buffer_rsrc(st, kGMap ? 0 : static_cast<int64_t>(seg_chunks) * kD * kD * 4);
    // the M half of a cotangent map sees dY = 0 (a per-workgroup, uniform branch)
    const bool use_dy = !kGMap || half == 1;

    // staging: thread tid moves row tid / 16, columns 4 (tid % 16) .. +3 of
    // each 16 x 64 tile, and rows tid / 16 + 16 q of W
    const int srow = tid >> 4;
    const int scol = 4 * (tid & 15);

    // prologue state of this staging thread (as in the bf16 kernel)
    const bool use_tok = kPro && pro.eta_tok != nullptr;
    const bool ln_q = kPro && pro.ln_q != nullptr;
    const bool ln_k = kPro && pro.ln_k != nullptr;
    const bool a_on = !kPro || !pro.read_start;      // uniform: the tril(Q K^T) term
    float* const etas = lds + (kGMap ? kOffEtaGMap : kOffEtaMain);
    float gmq[4], btq[4], gmk[4], btk[4];
    float xq[4] = {}, xk[4] = {}, rq = 1.f, rk = 1.f;
    float dgq[4] = {}, dbq[4] = {}, dgk[4] = {}, dbk[4] = {};
    if constexpr (kPro) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            gmq[e] = ln_q ? pro.ln_q[(2 * h) * kD + scol + e] : 1.f;
            btq[e] = ln_q ? pro.ln_q[(2 * h + 1) * kD + scol + e] : 0.f;
            gmk[e] = ln_k ? pro.ln_k[(2 * h) * kD + scol + e] : 1.f;
            btk[e] = ln_k ? pro.ln_k[(2 * h + 1) * kD + scol + e] : 0.f;
        }
    }
    const __amdgpu_buffer_rsrc_t r_eta =
        mfma::buffer_rsrc(use_tok ? pro.eta_tok + u * static_cast<int64_t>(T) : eta,
                   use_tok ? static_cast<int64_t>(T) * 4 : 0);
    const __amdgpu_buffer_rsrc_t r_deta =
        mfma::buffer_rsrc(use_tok && !kGMap ? deta_tok + u * static_cast<int64_t>(T) : eta,
                   use_tok && !kGMap ? static_cast<int64_t>(T) * 4 : 0);
    auto norm = [&](f32x4 x, const float (&gm)[4], const float (&bt)[4], bool valid,
                    float (&xh)[4], float& rstd) {
        const float f[4] = {x[0], x[1], x[2], x[3]};
        layernorm_row_keep<16, 4>(f, pro.ln_eps, valid, xh, rstd);
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            y[e] = valid ? xh[e] * gm[e] + bt[e] : 0.f;
        return y;
    };
    auto load_stage = [&](Stage<In>& x, int chunk, bool qdy, bool wst, bool with_v = true) {
        const int t = chunk * kB + srow;
        const int eb = (t * kD + scol) * 4;
        x.ok = t < T;
        if constexpr (kPro) {
            const float tok = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_eta, t * 4, 0, 0));
            x.eta = use_tok ? tok : (x.ok ? et : 0.f);
        }
        x.k = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r_k, eb, 0, 0));
        if (!kGMap && with_v) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                x.v[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    r_v, ((chunk * kB + 4 * g + r) * kD + 16 * w + c) * 4, 0, 0));
        }
        if (qdy) {
            x.q = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r_q, eb, 0, 0));
            x.dy = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r_dy, eb, 0, 0));
        }
        if (wst) {
            // chunk c0 - 1 (loaded ahead of the first chunk) falls outside: zeros
#pragma unroll
            for (int q = 0; q < 4; ++q)
                x.w[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    r_st, (((chunk - c0) * kD + srow + 16 * q) * kD + scol) * 4, 0, 0));
        }
    };
    auto store_stage = [&](const Stage<In>& x, int slot, bool qdy) {
        float* sl = lds + slot * kSlotFloats;
        f32x4 kx = Raw<In>::to_f32(x.k);
        if constexpr (kPro) {
            if (ln_k)
                kx = norm(kx, gmk, btk, x.ok, xk, rk);
            if ((tid & 15) == 0)
                etas[slot * kB + srow] = x.eta;
        }
        lds4(sl + kSlotK + srow * kP + scol, kx);
        if (qdy) {
            f32x4 qx = Raw<In>::to_f32(x.q);
            if constexpr (kPro) {
                if (ln_q)
                    qx = norm(qx, gmq, btq, x.ok, xq, rq);
            }
            lds4(sl + kSlotQ + srow * kP + scol, qx);
            lds4(sl + kSlotDY + srow * kP + scol, Raw<In>::to_f32(x.dy));
        }
    };
    // step sizes of rows 4g .. 4g + 3 of a slot (the head's without the prologue)
    auto rows_eta = [&](int slot) {
        if constexpr (kPro)
            return lds4(etas + slot * kB + 4 * g);
        else
            return f32x4{et, et, et, et};
    };
    auto store_w = [&](const Stage<In>& x) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            lds4(lds + kOffW + (srow + 16 * q) * kP + scol, x.w[q]);
    };

    // E_J = K W[:, J] - V[:, J] for this wave's columns J = w, from the
    // staged K of a slot, this lane's V entries and the W tiles Wt[i] (rows
    // 16 i + 4g + r)
    auto residual = [&](const float* sl, const float (&Wt)[4][4], const In (&vr)[4], f32x4 (&krow)[4]) {
        f32x4 acc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            acc[0][r] = -to_f(vr[r]);
        acc[1] = acc[2] = acc[3] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            krow[i] = lds4(sl + kSlotK + c * kP + 16 * i + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] = mfma(krow[i][r], Wt[i][r], acc[i]);
        return (acc[0] + acc[1]) + (acc[2] + acc[3]);
    };

    // ---------------- sweep 1: chunk-start states of the segment ----------------
    float Wt[4][4];
    if (!kGMap && c1 > c0) {
        const float* w0 = nseg > 1 ? wstart + (u * nseg + s) * kD * kD
                                   : W0 + (w0_per_batch ? u : h) * kD * kD;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Wt[i][r] = w0[(16 * i + 4 * g + r) * kD + 16 * w + c];
        // The chunks ahead in two rings of kAhead register sets (as in the
        // bf16 kernel): K of chunk ch + 1 in kring[(ch - c0) % kAhead], V of
        // chunk ch in vring[(ch - c0) % kAhead], each entry used in place;
        // rounds of kAhead chunks keep the indices static
        constexpr int kAhead = 4;
        Stage<In> kring[kAhead];
        In vring[kAhead][4];
        auto load_v = [&](In (&v)[4], int chunk) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    r_v, ((chunk * kB + 4 * g + r) * kD + 16 * w + c) * 4, 0, 0));
        };
        {
            Stage<In> first;
            load_stage(first, c0, false, false, false);
            store_stage(first, 0, false);
        }
#pragma unroll
        for (int q = 0; q < kAhead; ++q) {
            load_v(vring[q], c0 + q);
            load_stage(kring[q], c0 + 1 + q, false, false, false);
        }
        __syncthreads();
        // (`last`: the segment's last chunk, whose state is stored and nothing
        // more; a constant false in the full rounds)
        auto sweep1_step = [&](int ch, Stage<In>& knext, In (&vc)[4], bool last) {
            float* sc = st + static_cast<int64_t>(ch - c0) * kD * kD;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sc[(16 * i + 4 * g + r) * kD + 16 * w + c] = Wt[i][r];
            if (last)
                return;
            const float* sl = lds + ((ch - c0) & 1) * kSlotFloats;
            f32x4 krow[4];
            const f32x4 E = residual(sl, Wt, vc, krow);
            const f32x4 En = -(rows_eta((ch - c0) & 1) * E);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 acc = {Wt[i][0], Wt[i][1], Wt[i][2], Wt[i][3]};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc = mfma(sl[kSlotK + (4 * g + r) * kP + 16 * i + c], En[r], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Wt[i][r] = acc[r];
            }
            load_v(vc, ch + kAhead);
            store_stage(knext, (ch - c0 + 1) & 1, false);
            load_stage(knext, ch + 1 + kAhead, false, false, false);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        };
        int ch = c0;
        for (; ch + kAhead < c1; ch += kAhead) {
#pragma unroll
            for (int q = 0; q < kAhead; ++q)
                sweep1_step(ch + q, kring[q], vring[q], false);
        }
#pragma unroll
        for (int q = 0; q < kAhead; ++q) {
            if (ch + q >= c1)            // uniform
                break;
            sweep1_step(ch + q, kring[q], vring[q], ch + q + 1 == c1);
        }
        // the states just stored are read back below by other threads
        __threadfence();
        __syncthreads();
    }

    // ---------------- sweep 2: reverse over the chunks of the segment ----------------
    float Gt[4][4];
    if (kGMap) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Gt[i][r] = half == 0 && 16 * i + 4 * g + r == 16 * w + c ? 1.f : 0.f;
    } else {
        const float* g1 = nseg > 1 ? gend + (u * nseg + (nseg - 1 - s)) * kD * kD
                                   : dW_out + u * kD * kD;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Gt[i][r] = g1[(16 * i + 4 * g + r) * kD + 16 * w + c];
    }
    float deta_acc = 0.f;
    float* Es = lds + kOffE;
    float* Ps = lds + kOffP;
    float* Gs = lds + kOffG;
    float* dAs = lds + kOffDA + w * kB * kDAP;

    In vcur[4] = {};
    if (c1 > c0) {
        Stage<In> nx;
        load_stage(nx, c1 - 1, use_dy, !kGMap);
        store_stage(nx, 0, use_dy);
        if (!kGMap) {
            store_w(nx);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vcur[r] = nx.v[r];
        }
        __syncthreads();
    }
    for (int ch = c1 - 1; ch >= c0; --ch) {
        const int slot = (c1 - 1 - ch) & 1;
        const float* sl = lds + slot * kSlotFloats;
        Stage<In> nx;
        // (unconditional, so the loads keep exact wait counts: at the first
        // chunk it reads chunk c0 - 1, unused, zeros where it is outside)
        load_stage(nx, ch - 1, use_dy, !kGMap);

        // ---- phase A: columns J = w ----
        f32x4 krow[4];
        f32x4 E = {0.f, 0.f, 0.f, 0.f};
        f32x4 wrow[4];       // W[16 w + c][16 jb + 4g .. +3] for phase B
        if (!kGMap) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Wt[i][r] = lds[kOffW + (16 * i + 4 * g + r) * kP + 16 * w + c];
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
                wrow[jb] = lds4(lds + kOffW + (16 * w + c) * kP + 16 * jb + 4 * g);
            E = residual(sl, Wt, vcur, krow);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                krow[i] = lds4(sl + kSlotK + c * kP + 16 * i + 4 * g);
        }
        // P = A^T dY_J + K G'_J, A = tril(Q K^T) (S below holds S[t = 4g + r][s = c];
        // as an A operand it is A^T)
        f32x4 pacc[4] = {};
        float dyc[4] = {0.f, 0.f, 0.f, 0.f};
        if (use_dy) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dyc[r] = sl[kSlotDY + (4 * g + r) * kP + 16 * w + c];
        }
        if (use_dy && a_on) {
            f32x4 qrow[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                qrow[i] = lds4(sl + kSlotQ + c * kP + 16 * i + 4 * g);
            f32x4 sacc[4] = {};
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sacc[i] = mfma(qrow[i][r], krow[i][r], sacc[i]);
            f32x4 S = (sacc[0] + sacc[1]) + (sacc[2] + sacc[3]);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[r] = c <= 4 * g + r ? S[r] : 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                pacc[0] = mfma(S[r], dyc[r], pacc[0]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pacc[i] = mfma(krow[i][r], Gt[i][r], pacc[i]);
        const f32x4 P = (pacc[0] + pacc[1]) + (pacc[2] + pacc[3]);
        const f32x4 er = rows_eta(slot);                  // eta of rows 4g + r
        const f32x4 dE = -(er * P);
        if (!kGMap) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (use_tok) {
                    // -<P_t, E_t> over this wave's 16 columns
                    const float pe = group_sum<16>(P[r] * E[r]);
                    if (c == 0)
                        lds[kOffDeta + w * kB + 4 * g + r] = pe;
                } else {
                    deta_acc -= P[r] * E[r];
                }
                Es[(4 * g + r) * kP + 16 * w + c] = E[r];
                Ps[(4 * g + r) * kP + 16 * w + c] = P[r];
            }
        }
        // G' to LDS for phase B, then G = G' + Q^T dY + K^T dE (over tokens)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 acc = {Gt[i][0], Gt[i][1], Gt[i][2], Gt[i][3]};
            if (!kGMap) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Gs[(16 * i + 4 * g + r) * kP + 16 * w + c] = Gt[i][r];
            }
            if (use_dy) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc = mfma(sl[kSlotQ + (4 * g + r) * kP + 16 * i + c], dyc[r], acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc = mfma(sl[kSlotK + (4 * g + r) * kP + 16 * i + c], dE[r], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Gt[i][r] = acc[r];
        }

        if (!kGMap) {
            __syncthreads();
            // every wave has read W_c: the next chunk's W_c may replace it
            if (ch > c0)
                store_w(nx);
            // ---- phase B: input dims I = w ----
            // dA = -eta tril(dY E^T): lane holds dA[t = 4g + r][s = c]
            f32x4 dyrow[4], erow[4];
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                dyrow[jb] = lds4(sl + kSlotDY + c * kP + 16 * jb + 4 * g);
                erow[jb] = lds4(Es + c * kP + 16 * jb + 4 * g);
            }
            f32x4 dA = {0.f, 0.f, 0.f, 0.f};
            if (a_on) {
                f32x4 aacc[4] = {};
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int jb = 0; jb < 4; ++jb)
                        aacc[jb] = mfma(dyrow[jb][r], erow[jb][r], aacc[jb]);
                dA = (aacc[0] + aacc[1]) + (aacc[2] + aacc[3]);
                // dA[t][s] scales by eta_s (s = c)
                const float ec = kPro ? etas[slot * kB + c] : et;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dA[r] = c <= 4 * g + r ? -ec * dA[r] : 0.f;
                    dAs[(4 * g + r) * kDAP + c] = dA[r];
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
            // dQ_I = dY W[I, :]^T + dA K_I
            f32x4 qacc[4] = {};
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int jb = 0; jb < 4; ++jb)
                    qacc[jb] = mfma(dyrow[jb][r], wrow[jb][r], qacc[jb]);
            if (a_on) {
                const f32x4 darow = lds4(dAs + c * kDAP + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    qacc[0] = mfma(darow[r], sl[kSlotK + (4 * g + r) * kP + 16 * w + c], qacc[0]);
            }
            const f32x4 dq = (qacc[0] + qacc[1]) + (qacc[2] + qacc[3]);
            // dK_I = -eta (P W[I, :]^T + E G'[I, :]^T) + dA^T Q_I
            f32x4 kacc[4] = {};
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                const f32x4 prow = lds4(Ps + c * kP + 16 * jb + 4 * g);
                const f32x4 grow = lds4(Gs + (16 * w + c) * kP + 16 * jb + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    kacc[jb] = mfma(prow[r], wrow[jb][r], kacc[jb]);
                    kacc[jb] = mfma(erow[jb][r], grow[r], kacc[jb]);
                }
            }
            // rows t = 4g + r: the step sizes of phase A's rows
            f32x4 dk = -(er * ((kacc[0] + kacc[1]) + (kacc[2] + kacc[3])));
            if (a_on) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dk = mfma(dA[r], sl[kSlotQ + (4 * g + r) * kP + 16 * w + c], dk);
            }

            // stores: rows t = 16 ch + 4g + r, column 16 w + c (P of phase A is
            // this wave's column block, so dV = eta P needs no exchange)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int eb = ((ch * kB + 4 * g + r) * kD + 16 * w + c) * 4;   // past T: dropped
                if constexpr (!kPro) {
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dq[r]), r_dq, eb, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dk[r]), r_dk, eb, 0, 0);
                }
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(er[r] * P[r]), r_dv, eb, 0, 0);
            }
            if constexpr (kPro) {
                // the gradients of the normalised rows go to the staging
                // threads for the LayerNorm backward
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    lds[kOffDQ + (4 * g + r) * kP + 16 * w + c] = dq[r];
                    lds[kOffDK + (4 * g + r) * kP + 16 * w + c] = dk[r];
                }
                __syncthreads();
                float gq[4], gk[4];
                {
                    const f32x4 a = lds4(lds + kOffDQ + srow * kP + scol);
                    const f32x4 b = lds4(lds + kOffDK + srow * kP + scol);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        gq[e] = a[e];
                        gk[e] = b[e];
                    }
                }
                if (ln_q)
                    layernorm_row_backward<16, 4>(gq, xq, rq, gmq, dgq, dbq);
                if (ln_k)
                    layernorm_row_backward<16, 4>(gk, xk, rk, gmk, dgk, dbk);
                const int t = ch * kB + srow;
                const int eb = (t * kD + scol) * 4;                     // past T: dropped
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, f32x4{gq[0], gq[1], gq[2], gq[3]}), r_dq, eb, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, f32x4{gk[0], gk[1], gk[2], gk[3]}), r_dk, eb, 0, 0);
                if (use_tok) {
                    // the row's 16 lanes store the same sum (no branch)
                    const float* pd = lds + kOffDeta;
                    const float de = -((pd[srow] + pd[kB + srow]) + (pd[2 * kB + srow] + pd[3 * kB + srow]));
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(de), r_deta, t * 4, 0, 0);
                }
            }
        }
        if (ch > c0) {
            store_stage(nx, slot ^ 1, use_dy);
            if (!kGMap) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vcur[r] = nx.v[r];
            }
        }
        __syncthreads();
    }

    if (kGMap) {
        float* out = gmaps + ((u * (nseg - 1) + (nseg - 1 - s)) * 2 + half) * kD * kD;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                out[(16 * i + 4 * g + r) * kD + 16 * w + c] = Gt[i][r];
        return;
    }
    // dW0 of the chain is the cotangent of the first chunk-start state
    if (s == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dW0_chain[u * kD * kD + (16 * i + 4 * g + r) * kD + 16 * w + c] = Gt[i][r];
    }
    // this segment's share of deta: sum over the lanes, then over the waves
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        deta_acc += __shfl_xor(deta_acc, m);
    if (lane == 0)
        lds[kOffRed + w] = deta_acc;
    if constexpr (kPro) {
        // gamma, beta gradients: over the 4 rows of the wave (lanes 16 apart),
        // then over the waves; out[a][col], a = gamma_q, beta_q, gamma_k, beta_k
        float* lr = lds + kOffDQ;                        // [4 waves][4][64]
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v4[4] = {dgq[e], dbq[e], dgk[e], dbk[e]};
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float x = v4[a];
                x += __shfl_xor(x, 16);
                x += __shfl_xor(x, 32);
                if (lane < 16)
                    lr[(w * 4 + a) * kD + scol + e] = x;
            }
        }
        __syncthreads();
        dln_chain[(u * nseg + s) * (kDlnRows * kD) + tid] =
            (lr[tid] + lr[256 + tid]) + (lr[512 + tid] + lr[768 + tid]);
    } else {
        __syncthreads();
    }
    if (tid == 0)
        deta_chain[u * nseg + s] = (lds[kOffRed] + lds[kOffRed + 1]) + (lds[kOffRed + 2] + lds[kOffRed + 3]);
}

// Sums in a fixed order: dW0 over the batch (when W0 is shared by the batch),
// deta over the batch and the segments (always: eta is one value per head)
// and, with the prologue, the LayerNorm gamma, beta gradients over the batch
// and the segments (dln_q, dln_k [H][2][64] from dln_chain [B H][nseg][4][64]).
// The first w_blocks blocks give each dW0 element a thread (B independent
// loads); the rest give each deta and LayerNorm element a wave, whose lanes
// sum every 64th of its B * nseg terms and then combine by a butterfly: the
// terms load in parallel, and the order is the same on every run.
__global__ void __launch_bounds__(256)
linear_backward_reduce_kernel(const float* __restrict__ dW0_chain, const float* __restrict__ deta_chain,
                              int64_t B, int H, int nseg, int64_t w_blocks, float* __restrict__ dW0,
                              float* __restrict__ deta, const float* __restrict__ dln_chain,
                              float* __restrict__ dln_q, float* __restrict__ dln_k)
{
    const int64_t n = static_cast<int64_t>(H) * kD * kD;
    if (blockIdx.x < w_blocks) {
        const int64_t x = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
        if (x < n) {
            float acc = 0.f;
#pragma unroll 8
            for (int64_t bb = 0; bb < B; ++bb)
                acc += dW0_chain[bb * n + x];
            dW0[x] = acc;
        }
        return;
    }
    const int lane = threadIdx.x & 63;
    const int64_t task = (static_cast<int64_t>(blockIdx.x) - w_blocks) * 4 + (threadIdx.x >> 6);
    const int64_t terms = B * nseg;
    const float* src;
    int64_t stride;                      // between the terms of one (batch, segment) step
    float* out;
    if (task < H) {
        src = deta_chain + task * nseg;
        stride = 1;
        out = deta + task;
    } else {
        const int64_t e = task - H;      // [H][4][64]
        if (!dln_chain || e >= static_cast<int64_t>(H) * kDlnRows * kD)
            return;
        const int hh = static_cast<int>(e / (kDlnRows * kD));
        const int a = static_cast<int>(e / kD) % kDlnRows;   // gamma_q, beta_q, gamma_k, beta_k
        const int col = static_cast<int>(e % kD);
        out = a < 2 ? dln_q : dln_k;
        if (!out)
            return;
        out += (2 * hh + (a & 1)) * kD + col;
        src = dln_chain + static_cast<int64_t>(hh) * nseg * (kDlnRows * kD) + a * kD + col;
        stride = kDlnRows * kD;
    }
    // term q = bb nseg + sg sits at src + (bb H nseg + sg) stride
    float acc = 0.f;
    for (int64_t q = lane; q < terms; q += 64) {
        const int64_t bb = q / nseg, sg = q % nseg;
        acc += src[(bb * H * nseg + sg) * stride];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        acc += __shfl_xor(acc, m);
    if (lane == 0)
        *out = acc;
}

// workspace carve-up (floats): forward maps, start states, cotangent maps,
// end cotangents (only with segments), chunk-start states, per-chain dW0
// (shared W0 only), per-segment deta
using BwdWorkspace = BwdBuffers;

// One segment covers every chunk: seg_len = T rounded up to whole chunks.
SegmentPlan normalized(const LinearBwdArgs& a, SegmentPlan p)
{
    if (p.nseg <= 1) {
        p.nseg = 1;
        p.seg_len = (a.T + kB - 1) / kB * kB;
    }
    return p;
}

BwdWorkspace carve(const LinearBwdArgs& a, const SegmentPlan& p, void* base)
{
    const size_t units = static_cast<size_t>(a.B * a.H);
    const size_t st = kD * kD;
    const size_t seg_chunks = static_cast<size_t>(p.seg_len / kB);
    const size_t S = static_cast<size_t>(p.nseg);
    size_t o = 0;
    BwdWorkspace w{};
    float* f = static_cast<float*>(base);
    auto take = [&](size_t n) {
        float* r = f ? f + o : nullptr;
        o += (n + 63) / 64 * 64;       // 256-byte aligned pieces
        return r;
    };
    if (S > 1) {
        w.maps = take(units * (S - 1) * 2 * st);
        w.wstart = take(units * S * st);
        w.gmaps = take(units * (S - 1) * 2 * st);
        w.gend = take(units * S * st);
    }
    // chunk-start states: fp32 W for fp32 inputs; for bf16 the update
    // operands E' from which the bf16 kernel walks the states back (256
    // threads x 8 bytes per chunk: 512 floats' worth)
    w.states = take(units * S * seg_chunks * (a.dtype != 0 ? 512 : st));
    w.dw_chain = a.w0_per_batch ? a.dW0 : take(units * st);
    w.deta_chain = take(units * S);
    w.dln_chain = a.pro.active() ? take(units * S * kDlnRows * kD) : nullptr;
    w.bytes = o * sizeof(float);
    return w;
}

template <typename In, bool kGMap, bool kPro>
void launch_kernel(const LinearBwdArgs& a, const SegmentPlan& p, const BwdWorkspace& w, dim3 grid)
{
    const int lds = kPro ? (kGMap ? kProGMapLdsBytes : kProLdsBytes)
                         : (kGMap ? kGMapLdsBytes : kLdsBytes);
    hipLaunchKernelGGL((linear_backward_kernel<In, kGMap, kPro>), grid, dim3(kThreads), lds,
                       a.stream, static_cast<const In*>(a.Q), static_cast<const In*>(a.K),
                       static_cast<const In*>(a.V), a.W0, a.w0_per_batch, a.eta,
                       static_cast<int>(a.H), static_cast<int>(a.T), a.B * a.H,
                       static_cast<int>(p.seg_len), p.nseg, w.wstart, w.gend,
                       static_cast<const In*>(a.dY), a.dW_out, static_cast<In*>(a.dQ),
                       static_cast<In*>(a.dK), static_cast<In*>(a.dV), w.dw_chain, w.deta_chain,
                       w.states, w.gmaps, a.pro, a.deta_tok, w.dln_chain);
}

template <typename In, bool kGMap>
void launch_kernel(const LinearBwdArgs& a, const SegmentPlan& p, const BwdWorkspace& w, dim3 grid)
{
    if (a.pro.active())
        launch_kernel<In, kGMap, true>(a, p, w, grid);
    else
        launch_kernel<In, kGMap, false>(a, p, w, grid);
}

template <typename In>
hipError_t set_lds()
{
    const struct { const void* f; int bytes; } k[] = {
        {reinterpret_cast<const void*>(linear_backward_kernel<In, false, false>), kLdsBytes},
        {reinterpret_cast<const void*>(linear_backward_kernel<In, true, false>), kGMapLdsBytes},
        {reinterpret_cast<const void*>(linear_backward_kernel<In, false, true>), kProLdsBytes},
        {reinterpret_cast<const void*>(linear_backward_kernel<In, true, true>), kProGMapLdsBytes},
    };
    for (const auto& x : k) {
        const hipError_t e = hipFuncSetAttribute(x.f, hipFuncAttributeMaxDynamicSharedMemorySize, x.bytes);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace

bool linear_backward_supports(const LinearBwdArgs& a)
{
    // per-chain byte offsets are 32-bit (fp32 rows of 256 bytes; the forward
    // maps and start-state kernels it launches have the same bound)
    const int64_t max_tokens = (int64_t{1} << 31) / (kD * 4) - kB * 64;
    return a.d == kD && a.b == kB && a.T <= max_tokens;
}

size_t linear_backward_workspace_bytes(const LinearBwdArgs& a, const SegmentPlan& p)
{
    return carve(a, normalized(a, p), nullptr).bytes;
}

hipError_t launch_linear_backward(const LinearBwdArgs& a, const SegmentPlan& plan, void* workspace)
{
    const int64_t units = a.B * a.H;
    const SegmentPlan p = normalized(a, plan);
    const BwdWorkspace w = carve(a, p, workspace);
    const bool bf16 = a.dtype != 0;
    hipError_t e = bf16 ? hipSuccess : set_lds<float>();
    if (e != hipSuccess)
        return e;
    if (units > 0 && p.nseg > 1) {
        // start state of every segment: the forward's maps and composition
        LinearArgs fa{a.Q, a.K, a.V, a.dtype, a.W0, a.w0_per_batch, a.eta, a.B, a.H, a.T,
                      a.d, a.b, nullptr, nullptr, a.stream};
        fa.pro = a.pro;
        SegmentPlan fp = p;
        fp.maps = w.maps;
        fp.wstart = w.wstart;
        fp.starts_only = true;
        e = bf16 ? launch_linear_mfma(fa, fp) : launch_linear_mfma_f32(fa, fp);
        if (e != hipSuccess)
            return e;
        // end cotangent of every segment: cotangent maps, then the same
        // composition run from dW_out through the segments in reverse
        const dim3 mgrid(static_cast<unsigned>(placed_grid(units, 2 * (p.nseg - 1))));
        if (bf16) {
            e = launch_linear_backward_bf16(a, p, true, w, mgrid);
        } else {
            launch_kernel<float, true>(a, p, w, mgrid);
            e = hipGetLastError();
        }
        if (e != hipSuccess)
            return e;
        const LinearArgs ga{a.Q, a.K, a.V, a.dtype, a.dW_out, 1, a.eta, a.B, a.H, a.T,
                            a.d, a.b, nullptr, nullptr, a.stream};
        SegmentPlan gp = p;
        gp.maps = w.gmaps;
        gp.wstart = w.gend;
        e = launch_linear_combine(ga, gp);
        if (e != hipSuccess)
            return e;
    }
    if (units > 0) {
        const dim3 grid(static_cast<unsigned>(p.nseg > 1 ? placed_grid(units, p.nseg) : units));
        if (bf16) {
            e = launch_linear_backward_bf16(a, p, false, w, grid);
        } else {
            launch_kernel<float, false>(a, p, w, grid);
            e = hipGetLastError();
        }
        if (e != hipSuccess)
            return e;
    }
    const int64_t w_blocks = a.w0_per_batch ? 0 : (a.H * kD * kD + 255) / 256;
    const int64_t wave_tasks = a.H + (a.pro.active() ? a.H * kDlnRows * kD : 0);
    hipLaunchKernelGGL(linear_backward_reduce_kernel,
                       dim3(static_cast<unsigned>(w_blocks + (wave_tasks + 3) / 4)), dim3(256), 0,
                       a.stream, w.dw_chain, w.deta_chain, a.B, static_cast<int>(a.H), p.nseg,
                       w_blocks, a.dW0, a.deta, w.dln_chain, a.dln_q, a.dln_k);
    return hipGetLastError();
}

}  // namespace ttt
