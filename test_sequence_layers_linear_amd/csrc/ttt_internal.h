// ttt_internal.h -- declarations shared by the kernels and the C-ABI layer of
// libttt.so.  Not part of the public ABI (that is include/ttt.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

// Maximum LDS one workgroup may use on gfx950.
constexpr int kMaxLdsBytes = 160 * 1024;
// MI355X's last-level (Infinity) cache
constexpr int64_t kLastLevelCacheBytes = int64_t{256} << 20;

// ---------------------------------------------------------------------------
// element access: Q/K/V/Y are fp32 or bf16 (stored as raw 16-bit patterns)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, int64_t i)
{
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ void store_elem(float* p, int64_t i, float x) { p[i] = x; }
// fp32 -> bf16, round to nearest even (lowers to v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x)
{
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ void store_elem(uint16_t* p, int64_t i, float x)
{
    p[i] = f32_to_bf16_bits(x);
}

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }

// ---------------------------------------------------------------------------
// launchers (each returns hipSuccess or the launch error)
// ---------------------------------------------------------------------------
// Optional input prologue of the TTT-Linear MFMA kernels: LayerNorm of the q
// and k rows over the head dim (per-head gamma, beta; biased variance) and a
// step size per token instead of the head's.  All null: the plain scan.
struct Prologue {
    const float* eta_tok = nullptr;   // [B][H][T]
    const float* ln_q = nullptr;      // [H][2][d]: gamma row, then beta row
    const float* ln_k = nullptr;
    float ln_eps = 1e-5f;
    int read_start = 0;               // 1: tokens read out with the chunk-start W
    bool active() const { return eta_tok || ln_q || ln_k || read_start; }
};

struct LinearArgs {
    const void* Q; const void* K; const void* V; int dtype;
    const float* W0; int w0_per_batch; const float* eta;
    int64_t B, H, T; int d, b;
    void* Y; float* W_out; hipStream_t stream;
    Prologue pro{};
};

// Sum over each aligned group of kLanes (8 or 16) lanes, every lane of the
// group receiving it, with DPP lane permutes (no LDS round trip): quad
// xor 1, quad xor 2, then the half-row mirror (lane i <-> 7 - i: the other
// quad) and, for 16 lanes, the row mirror (i <-> 15 - i: the other half).
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl,
                                                              0xf, 0xf, true));
}
template <int kLanes>
__device__ __forceinline__ float group_sum(float x)
{
    static_assert(kLanes == 8 || kLanes == 16, "8 or 16 lanes");
    x += dpp_mov<0xb1>(x);      // quad_perm [1, 0, 3, 2]
    x += dpp_mov<0x4e>(x);      // quad_perm [2, 3, 0, 1]
    x += dpp_mov<0x141>(x);     // row_half_mirror
    if (kLanes == 16)
        x += dpp_mov<0x140>(x); // row_mirror
    return x;
}

// LayerNorm of one 64-element row spread over kLanes consecutive lanes (kN
// elements each, all lanes of the wave active): mean and biased variance
// (two passes), then (x - mean) / sqrt(var + eps) * gamma + beta; a row that
// is not `valid` (past the sequence end) becomes 0.
template <int kLanes, int kN>
__device__ __forceinline__ void layernorm_row(float (&x)[kN], const float (&gm)[kN],
                                              const float (&bt)[kN], float eps, bool valid)
{
    static_assert(kLanes * kN == 64, "one 64-element row");
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < kN; ++i)
        sum += x[i];
    const float mean = group_sum<kLanes>(sum) * (1.0f / 64.0f);
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < kN; ++i)
        sq += (x[i] - mean) * (x[i] - mean);
    const float rstd = rsqrtf(group_sum<kLanes>(sq) * (1.0f / 64.0f) + eps);
#pragma unroll
    for (int i = 0; i < kN; ++i)
        x[i] = valid ? (x[i] - mean) * rstd * gm[i] + bt[i] : 0.f;
}

// The same LayerNorm keeping what its backward needs: xh = (x - mean) * rstd
// (0 for a row that is not `valid`) and rstd.
template <int kLanes, int kN>
__device__ __forceinline__ void layernorm_row_keep(const float (&x)[kN], float eps, bool valid,
                                                   float (&xh)[kN], float& rstd)
{
    static_assert(kLanes * kN == 64, "one 64-element row");
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < kN; ++i)
        sum += x[i];
    const float mean = group_sum<kLanes>(sum) * (1.0f / 64.0f);
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < kN; ++i)
        sq += (x[i] - mean) * (x[i] - mean);
    rstd = rsqrtf(group_sum<kLanes>(sq) * (1.0f / 64.0f) + eps);
#pragma unroll
    for (int i = 0; i < kN; ++i)
        xh[i] = valid ? (x[i] - mean) * rstd : 0.f;
}

// Backward of layernorm_row for one row spread like it: given the gradient
// gy of the normalised row y = xh * gamma + beta, returns the gradient of the
// raw row in gy and adds gy * xh, gy to the gamma, beta sums:
//     dxh = gy gamma,  dx = rstd (dxh - mean(dxh) - xh mean(dxh xh)).
template <int kLanes, int kN>
__device__ __forceinline__ void layernorm_row_backward(float (&gy)[kN], const float (&xh)[kN],
                                                       float rstd, const float (&gm)[kN],
                                                       float (&dgamma)[kN], float (&dbeta)[kN])
{
    float dxh[kN];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < kN; ++i) {
        dgamma[i] += gy[i] * xh[i];
        dbeta[i] += gy[i];
        dxh[i] = gy[i] * gm[i];
        s1 += dxh[i];
        s2 += dxh[i] * xh[i];
    }
    s1 = group_sum<kLanes>(s1) * (1.0f / 64.0f);
    s2 = group_sum<kLanes>(s2) * (1.0f / 64.0f);
#pragma unroll
    for (int i = 0; i < kN; ++i)
        gy[i] = rstd * (dxh[i] - s1 - xh[i] * s2);
}

struct MlpArgs {
    const void* Q; const void* K; const void* V; int dtype;
    const float* W1_0; const float* W2_0; int w0_per_batch; const float* eta;
    int64_t B, H, T; int d, m, b;
    void* Y; float* W1_out; float* W2_out; hipStream_t stream;
};

struct DecodeArgs {
    const void* q; const void* k; const void* v; int dtype;
    float* W; const float* eta; int64_t B, H; int d;
    void* y; hipStream_t stream;
    Prologue pro{};                   // eta_tok is [B][H] here (one token)
};

// Generic kernels: any supported d and b, fp32 arithmetic, state in LDS
// (linear) or in the output buffers (MLP).  LDS bytes they need:
size_t linear_generic_lds_bytes(int d, int b);
size_t mlp_generic_lds_bytes(int d, int m, int b);
hipError_t launch_linear_generic(const LinearArgs& a);
hipError_t launch_mlp_generic(const MlpArgs& a);

// Sequence-segment split of the TTT-Linear scan.  Each chunk maps the state
// affinely, W' = (I - eta K^T K) W + eta K^T V, so a run of chunks does too:
// W_end = M W_start + N.  With nseg > 1 the tokens of a chain are cut into
// segments of seg_len tokens (a multiple of the chunk size); one launch
// computes (M, N) of every segment but the last into `maps`
// ([B H][nseg - 1][2][d][d] fp32), a second composes them into the start
// state of every segment (`wstart`, [B H][nseg][d][d], wstart[.][0] = W0),
// and a third runs every segment's scan from its start state.
struct SegmentPlan {
    int nseg = 1;
    int64_t seg_len = 0;        // tokens of segments 1 .. nseg - 1
    int64_t first_len = 0;      // tokens of segment 0 (0: seg_len)
    float* maps = nullptr;
    float* wstart = nullptr;
    bool starts_only = false;   // maps and start states only, no segment scans
    // segment 0 scanned beside the maps of segments 1 .. nseg - 2 (bf16
    // TTT-Linear, with or without the prologue): no map of segment 0, and the
    // composition starts from its end state
    bool fused = false;
    int64_t first() const { return first_len > 0 ? first_len : seg_len; }
};

// Block id -> (chain u, block s of the chain) for nb blocks per chain.  With
// at least 8 chains every block of chain u gets id = u (mod 8): workgroups
// are dispatched to the 8 XCDs round robin, so they all share XCD u % 8 and
// its L2 (grid 8 nb ceil(units / 8); ids with u >= units do nothing).  With
// fewer chains that would leave XCDs idle, so blocks are numbered plainly.
__device__ __forceinline__ void xcd_block(int id, int nb, int64_t units, int64_t& u, int& s)
{
    if (units < 8) {
        u = id / nb;
        s = id % nb;
        return;
    }
    const int t = id >> 3;
    u = 8 * static_cast<int64_t>(t / nb) + (id & 7);
    s = t % nb;
}
__host__ __device__ inline int64_t placed_grid(int64_t units, int nb)
{
    return units < 8 ? units * nb : 8 * nb * ((units + 7) / 8);
}
hipError_t launch_linear_combine(const LinearArgs& a, const SegmentPlan& p);
size_t linear_combine_lds_bytes(int nseg);
// most segments per chain (the combine step keeps every start state in LDS)
constexpr int kMaxSegments = 30;   // with the ring's spare slots: 36 x 4352 B of LDS

// MFMA kernels for the d = 64, b = 16 (and m = 256) shapes: bf16 inputs on
// bf16 MFMA, fp32 inputs on fp32 MFMA.  Latencies (us) that size the segment
// split: forward chunk, map chunk, one step of the start-state composition,
// and the fixed cost of the two extra launches.
struct SegmentCosts {
    double fwd, map, apply, launch;
    int map_blocks_per_segment;       // workgroups of the maps launch per segment
    int scan_blocks_per_segment = 1;  // workgroups of the scan launch per segment
    int map_blocks_per_cu = 1;        // maps workgroups one CU may hold
};
bool linear_mfma_supports(const LinearArgs& a);
hipError_t launch_linear_mfma(const LinearArgs& a, const SegmentPlan& p);
bool linear_mfma_f32_supports(const LinearArgs& a);
hipError_t launch_linear_mfma_f32(const LinearArgs& a, const SegmentPlan& p);
// bf16: chunk costs of the current scan and maps on MI355X, and the fixed
// cost of a segmented call (the extra launches, the composition's launch and
// the launches' tails), fitted to B8 H12 T2048 (unsegmented 40 us, fused with
// 3 segments 46 us) and B2 H24 T32768 (unfused with 5 segments 237-255 us,
// fused with 6 segments 227-230 us)
constexpr SegmentCosts kLinearBf16Costs{0.32, 0.25, 0.60, 18.0, 1};
// a chunk of the 12-wave staged scan (the fused layout's segment 0) over one
// of the plain 4-wave scan: 163 against 140 us per segment on B2 H24 T32768
constexpr double kStagedScanFactor = 1.16;
constexpr SegmentCosts kLinearF32Costs{1.38, 0.90, 0.60, 8.5, 2};
// fp32 Q/K/V with each chain's W split by columns over 4 workgroups
// (ttt_linear_cols_f32.hip, with or without the prologue): used while the chains'
// 4 workgroups each fit the GPU's CUs, where it cuts a chunk's latency.
bool linear_cols_f32_supports(const LinearArgs& a);
hipError_t launch_linear_cols_f32(const LinearArgs& a, const SegmentPlan& p);
constexpr int kColsSlices = 4;
constexpr SegmentCosts kLinearF32ColsCosts{0.79, 0.55, 0.90, 4.5, 2 * kColsSlices, kColsSlices, 2};
bool mlp_mfma_supports(const MlpArgs& a);
hipError_t launch_mlp_mfma(const MlpArgs& a);

// Backward of the TTT-Linear scan (d = 64, b = 16), optionally cut into
// sequence segments like the forward: the forward maps give every segment's
// start state, cotangent maps composed from dW_out backwards give every
// segment's end cotangent, and then all segments run at once.  The workspace
// holds those maps and states, the recomputed chunk-start states, and
// per-chain dW0 (shared W0) and per-segment deta.
// With the prologue on, Q and K are the raw rows (LayerNorm'd inside), the
// step sizes are per token when pro.eta_tok is set (their gradients go to
// deta_tok [B][H][T]; deta is then 0), and dln_q, dln_k [H][2][d] receive the
// gradients of the LayerNorm gamma, beta rows (when ln_q, ln_k are set).
struct LinearBwdArgs {
    const void* Q; const void* K; const void* V; int dtype;
    const float* W0; int w0_per_batch; const float* eta;
    int64_t B, H, T; int d, b;
    const void* dY; const float* dW_out;
    void* dQ; void* dK; void* dV; float* dW0; float* deta; hipStream_t stream;
    Prologue pro{};
    float* deta_tok = nullptr;
    float* dln_q = nullptr;
    float* dln_k = nullptr;
};
// Device buffers of one backward call (carved from the stream's workspace;
// the segment maps and states only with several segments; the per-segment
// LayerNorm gradient sums only with the prologue).
struct BwdBuffers {
    float *maps, *wstart, *gmaps, *gend, *states, *dw_chain, *deta_chain, *dln_chain;
    size_t bytes;
};
// Per-segment LayerNorm gradient sums: [B H][nseg][4][64] floats in the order
// gamma_q, beta_q, gamma_k, beta_k.
constexpr int kDlnRows = 4;
// bf16 inputs on bf16 MFMA (ttt_linear_backward_bf16.hip): the cotangent maps
// (gmap) or the segment backward, on the given grid.
hipError_t launch_linear_backward_bf16(const LinearBwdArgs& a, const SegmentPlan& p, bool gmap,
                                       const BwdBuffers& b, dim3 grid);
bool linear_backward_supports(const LinearBwdArgs& a);
// Latencies (us) that size the backward's segment split: backward chunk
// (one workgroup on a CU), forward map chunk, cotangent map chunk, one
// composition step, the fixed cost of the four extra launches; workgroups per
// segment of the forward maps launch (the cotangent maps always take two);
// segment-backward workgroups a CU may hold, and the slowdown of each per
// extra workgroup per CU (measured on MI355X: the bf16 kernel's 32 KB of LDS
// let two share a CU, each 1.7x slower at 1.9 per CU; the fp32 kernel gains
// nothing from sharing); maps workgroups a CU may hold.  The bf16 figures
// are a least-squares fit to forced segment counts on MI355X (B8 H12 T2048:
// 173, 167, 176, 181, 207 us at 2-6 segments; B2 H24 T32768: 1111, 1007,
// 906 us at 6, 8, 10), where the composition step also stands for every
// other cost that grows with the segment count.
struct BwdCosts {
    double bwd, fmap, gmap, apply, launch;
    int fmap_blocks_per_segment;
    int max_per_cu;
    double share;
    int maps_per_cu;
};
constexpr BwdCosts kLinearBwdF32Costs{5.2, 0.9, 1.5, 0.6, 20.0, 2, 1, 0.0, 2};
constexpr BwdCosts kLinearBwdBf16Costs{1.64, 0.27, 0.62, 10.0, 5.3, 1, 2, 0.88, 4};
// the same with the input prologue (LayerNorm of q, k, per-token step sizes:
// a dearer chunk, so more segments pay), fitted to B8 H12 T2048 at 1-6
// segments (367, 311, 265, 247, 238, 285 us) and B2 H24 T32768 at 8 and 10
// (1433, 1233 us)
constexpr BwdCosts kLinearBwdBf16ProCosts{2.87, 0.47, 1.10, 16.7, 0.0, 1, 2, 0.074, 4};
size_t linear_backward_workspace_bytes(const LinearBwdArgs& a, const SegmentPlan& p);
hipError_t launch_linear_backward(const LinearBwdArgs& a, const SegmentPlan& p, void* workspace);

// Decode step.
hipError_t launch_decode(const DecodeArgs& a);

// TTT-Linear with momentum gradient descent (ttt_momentum.hip): grad_mode 0
// takes each token's gradient at the current weights (exact token steps),
// 1 at the chunk start; M0 null means a zero start momentum.
struct MomentumArgs {
    const void* Q; const void* K; const void* V; int dtype;
    const float* W0; int w0_per_batch; const float* M0;
    const float* eta; const float* beta; int grad_mode;
    int64_t B, H, T; int d, b;
    void* Y; float* W_out; float* M_out; hipStream_t stream;
};
size_t momentum_generic_lds_bytes(int d, int b);
hipError_t launch_momentum_generic(const MomentumArgs& a);
// bf16 d = 64, b = 16 on MFMA (ttt_momentum_mfma.hip).  Exact token steps
// need a workspace of momentum_mfma_workspace_bytes for the per-chunk
// triangular inverses.
bool momentum_mfma_supports(const MomentumArgs& a);
int64_t momentum_mfma_workspace_bytes(const MomentumArgs& a, int nseg);
hipError_t launch_momentum_mfma(const MomentumArgs& a, void* workspace, int nseg, int64_t seg_len);
// Start states [W; M] of the segments of a segmented momentum scan from the
// segments' maps (ttt_linear_combine.hip): xstart [units][nseg][2d][d].
hipError_t launch_momentum_combine(const MomentumArgs& a, const float* maps, int nseg,
                                   float* xstart);
size_t momentum_combine_lds_bytes(int nseg);
// most segments per chain of the momentum scan (its start states, 2d rows
// each, stay in the combine's LDS)
constexpr int kMaxMomentumSegments = 12;
// per-chunk latencies (us) of the bf16 momentum scan and its maps (three
// workgroups per segment: the W and M basis columns and the V columns)
constexpr SegmentCosts kMomentumExactCosts{0.50, 0.50, 1.2, 10.0, 3, 1, 2};
constexpr SegmentCosts kMomentumChunkStartCosts{0.43, 0.43, 1.2, 10.0, 3, 1, 2};

}  // namespace ttt
