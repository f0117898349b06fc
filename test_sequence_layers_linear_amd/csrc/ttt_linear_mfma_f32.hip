// ttt_linear_mfma_f32.hip -- TTT-Linear dual-form scan on fp32 MFMA for fp32
// Q/K/V, head dim d = 64, mini-batch b = 16, fp32 fast weights.
//
// Same recurrence and work split as the bf16 kernel (one workgroup of 4 waves
// per (batch, head) chain, wave w owns the 16 output columns [16w, 16w + 16)
// of W), with every product in fp32 on v_mfma_f32_16x16x4_f32:
//     E' = eta (V - K W),   Y = Q W + tril(Q K^T) E',   W = W + K^T E'
// ("Test-Time Training Layers: How Inner-Loop Gradient Descent Replaces the
// Transformer KV Cache ...", section "Hardware Parallelization: The Dual Form
// and Mini-Batch GPU Acceleration").
//
// 16x16x4 fp32 layouts (lane l, c = l % 16, g = l / 16):
//   A: lane holds A[c][k = g];  B: lane holds B[k = g][c];
//   C/D: lane holds rows 4g..4g+3 of column c.
// W slice: four 16-row accumulator tiles mt; row 4g + r of tile mt is input
// index i = 16g + 4mt + r.  A product contracting over i in 16 k-steps
// ks = 0..15 with k-slot g <-> i = 16g + ks then takes as its W operand the
// register Wacc[ks / 4][ks % 4] itself (no conversion, no data movement), and
// the K or Q operand of lane (c, g) for all 16 k-steps is the 64-byte row
// segment [16g, 16g + 16) of token c.  Products:
//   R   = -V + K W_J   : V^T read from LDS straight into the accumulator
//   S^T = K Q^T        : C layout = B layout of the E'^T S^T product
//   Y^T = W_J^T Q^T + E'^T S^T (masked)
//   W  += K^T E'       : 4 k-steps over tokens t = 4g + q; E' register q is
//                        the B operand and K^T rows come from LDS
// Each product over i runs as 4 independent accumulators (k-steps ks mod 4)
// that are summed at the end, so the 16 MFMAs of a product form 4 short
// dependency chains instead of one long one.
//
// Memory: as in the bf16 kernel, with a stage of one chunk: wave w loads rows
// [4w, 4w + 4) of the chunk's K, Q and V (three 1 KB row blocks, 16 bytes per
// lane) two register sets ahead, then writes them into a 3-slot LDS ring
// holding K and Q row-major (16-byte segments XOR-swizzled by row) and K^T,
// V^T (token-contiguous rows, segments swizzled by row group).  One barrier
// per chunk.  Every product is a 16x16x4 fp32 MFMA, so accumulation chains
// never mix MFMA shapes.
#include "ttt_mfma_ops.h"

namespace ttt {
namespace {

constexpr int kD = 64;
constexpr int kB = 16;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSet = 6;                 // chunks per register set (two sets)
constexpr int kSlots = 3;

constexpr int kRowBytes = kD * 4;                    // 256
constexpr int kOffK = 0;
constexpr int kOffQ = kOffK + kB * kRowBytes;        // 4096
constexpr int kOffKt = kOffQ + kB * kRowBytes;       // 8192  [64 i][16 t] fp32
constexpr int kOffVt = kOffKt + kD * kB * 4;         // 12288 [64 j][16 t] fp32
constexpr int kSlotBytes = kOffVt + kD * kB * 4;     // 16384

static_assert((2 * kSet) % kSlots == 0, "slot index must be static inside the loop");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// K, Q tiles: row r (token), 16-byte segment s in [0, 16)
__device__ __forceinline__ int swz_row(int r, int s) { return r * kRowBytes + ((s ^ (r & 15)) << 4); }
// K^T, V^T tiles: row x (input / output index), 16-byte segment s in [0, 4)
// (4 tokens each); the segment is swizzled by the row group so that 8 lanes
// reading segment s of 8 rows ρ hit 8 different bank groups.
__device__ __forceinline__ int swz_kt(int i, int s) { return i * 64 + ((s ^ ((i >> 4) & 3)) << 4); }
__device__ __forceinline__ int swz_vt(int j, int s) { return j * 64 + ((s ^ ((j >> 2) & 3)) << 4); }

struct StageRegs {
    u32x4 k, q, v;
    uint32_t eta;      // step size of this lane's token (prologue only)
};

// Row of W held in register r of accumulator tile mt by lane group g.
__device__ __forceinline__ int wrow(int mt, int m) { return 16 * (m >> 2) + 4 * mt + (m & 3); }


// kMaps = false: the scan of segment s of a chain (Y rows of the segment; the
//   last segment also writes W_out), started from W0 (one segment) or from
//   the segment's start state in wstart.
// kMaps = true: the affine map W_end = M W_start + N of segment s < nseg - 1;
//   block half 0 runs the scan from W = I with V = 0 (giving M), half 1 from
//   W = 0 with the segment's V (giving N).  No Q, no Y.  (The two halves run
//   as separate workgroups: this kernel is bound by the CU's fp32 MFMA rate,
//   so sharing one CU would halve each half's speed.)
// With nseg > 1 the blocks of chain u all run on XCD u % 8 (see xcd_block),
// so the maps, start states and scans of a chain meet in one L2.
// kPro: the input prologue (Prologue in ttt_internal.h) is applied while the
//   inputs are staged: K and Q rows LayerNorm'd over the head dim, and each
//   token's step size written next to the chunk in LDS, where it scales its
//   row of the residual: E'[t] = -eta_t R[t] (the head's eta when no
//   per-token step sizes are given); with read_start every token reads out
//   with the chunk-start W (the tril term is dropped).
template <bool kMaps, bool kPro>
__global__ void __launch_bounds__(kThreads, 1)
linear_mfma_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                       const float* __restrict__ V, const float* W0, int w0_per_batch,
                       const float* __restrict__ eta, int H, int T, int64_t units, int seg_len,
                       int nseg, float* maps, const float* wstart, float* __restrict__ Y,
                       float* W_out, Prologue pro)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int col = 16 * w + c;

    int64_t u = blockIdx.x;
    int s = 0, half = 0;
    if (nseg > 1) {
        xcd_block(blockIdx.x, kMaps ? 2 * (nseg - 1) : nseg, units, u, s);
        if (u >= units)                  // padding of the XCD placement
            return;
        if (kMaps) {
            half = s & 1;
            s >>= 1;
        }
    }
    const int h = static_cast<int>(u % H);
    const float et = eta[h];
    const int t_begin = s * seg_len;
    const int t_len = min(seg_len, T - t_begin);
    // map j of chain u: M at maps + (u (nseg - 1) + j) 2 64 64, N right after
    auto map_ptr = [&](int j) { return maps + ((u * (nseg - 1) + j) * 2) * kD * kD; };

    // Wacc[mt][r] = W[16g + 4mt + r][col]
    f32x4 Wacc[4];
    if (kMaps) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Wacc[mt][r] = (half == 0 && wrow(mt, 4 * g + r) == col) ? 1.0f : 0.0f;
    } else {
        const float* w0 = nseg > 1 ? wstart + (u * nseg + s) * kD * kD
                                   : W0 + (w0_per_batch ? u : h) * kD * kD;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Wacc[mt][r] = w0[wrow(mt, 4 * g + r) * kD + col];
    }

    const int64_t base = (u * static_cast<int64_t>(T) + t_begin) * kD;
    const int64_t seg_bytes = static_cast<int64_t>(t_len) * kD * 4;
    const __amdgpu_buffer_rsrc_t rq = mfma::buffer_rsrc(Q + base, kMaps ? 0 : seg_bytes);
    const __amdgpu_buffer_rsrc_t rk = mfma::buffer_rsrc(K + base, seg_bytes);
    const __amdgpu_buffer_rsrc_t rv = mfma::buffer_rsrc(V + base, (kMaps && half == 0) ? 0 : seg_bytes);
    const __amdgpu_buffer_rsrc_t ry = mfma::buffer_rsrc(Y + base, kMaps ? 0 : seg_bytes);

    const int nchunks = (t_len + kB - 1) / kB;
    // a slot also holds the chunk's 16 step sizes when the prologue is on
    constexpr int kSlotB = kPro ? kSlotBytes + kB * 4 : kSlotBytes;
    constexpr int kSetK = kSet;
    static_assert((2 * kSetK) % kSlots == 0, "slot index must be static inside the loop");
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // staging: lane l of wave w holds row 4w + l / 16, 16-byte segment l % 16
    const int st_row = 4 * w + (lane >> 4);
    const int st_seg = lane & 15;
    // prologue: LayerNorm gamma, beta of this lane's 4 columns 4 st_seg .. +3
    const bool use_tok = kPro && pro.eta_tok != nullptr;
    const bool ln_k = kPro && pro.ln_k != nullptr;
    const bool ln_q = kPro && !kMaps && pro.ln_q != nullptr;
    float gk[4], bk[4], gq[4], bq[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        gk[e] = ln_k ? pro.ln_k[(2 * h) * kD + 4 * st_seg + e] : 1.f;
        bk[e] = ln_k ? pro.ln_k[(2 * h + 1) * kD + 4 * st_seg + e] : 0.f;
        gq[e] = ln_q ? pro.ln_q[(2 * h) * kD + 4 * st_seg + e] : 1.f;
        bq[e] = ln_q ? pro.ln_q[(2 * h + 1) * kD + 4 * st_seg + e] : 0.f;
    }
    const __amdgpu_buffer_rsrc_t reta =
        mfma::buffer_rsrc(use_tok ? pro.eta_tok + u * static_cast<int64_t>(T) + t_begin : eta,
                   use_tok ? static_cast<int64_t>(t_len) * 4 : 0);
    auto load_stage = [&](StageRegs& o, int chunk) {
        const int off = (chunk * kB + st_row) * kRowBytes + st_seg * 16;
        o.k = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        if (!kMaps)
            o.q = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
        o.v = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
        if (use_tok)
            o.eta = __builtin_amdgcn_raw_buffer_load_b32(reta, (chunk * kB + st_row) * 4, 0, 0);
    };
    // LayerNorm of a staged row segment (16 lanes per row)
    auto norm = [&](u32x4 x, const float (&gm)[4], const float (&bt)[4], bool valid) {
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            f[e] = __uint_as_float(x[e]);
        layernorm_row<16, 4>(f, gm, bt, pro.ln_eps, valid);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            x[e] = __float_as_uint(f[e]);
        return x;
    };
    // LayerNorm a chunk's rows in their registers, at the end of the chunk
    // before the one that writes them to LDS: after that chunk's products, so
    // that the scheduler can overlap the two
    auto prep = [&](StageRegs& o, int chunk) {
        if constexpr (kPro) {
            const bool valid = chunk * kB + st_row < t_len;
            if (ln_k)
                o.k = norm(o.k, gk, bk, valid);
            if (ln_q)
                o.q = norm(o.q, gq, bq, valid);
        }
    };
    auto write_stage = [&](const StageRegs& o, int slot) {
        unsigned char* sl = lds + slot * kSlotB;
        if constexpr (kPro) {
            if (st_seg == 0)
                *reinterpret_cast<float*>(sl + kSlotBytes + 4 * st_row) =
                    use_tok ? __uint_as_float(o.eta) : et;
        }
        *reinterpret_cast<u32x4*>(sl + kOffK + swz_row(st_row, st_seg)) = o.k;
        if (!kMaps)
            *reinterpret_cast<u32x4*>(sl + kOffQ + swz_row(st_row, st_seg)) = o.q;
        // transposed copies: element e of this segment is index 4 st_seg + e;
        // token st_row sits at position st_row % 4 of 16-byte segment st_row / 4
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int x = 4 * st_seg + e;
            *reinterpret_cast<uint32_t*>(sl + kOffKt + swz_kt(x, st_row >> 2) + 4 * (st_row & 3)) = o.k[e];
            *reinterpret_cast<uint32_t*>(sl + kOffVt + swz_vt(x, st_row >> 2) + 4 * (st_row & 3)) = o.v[e];
        }
    };

    struct ChunkOps {
        f32x4 k[4];        // K[t = c][16g + 4x .. +3], x = 0..3
        f32x4 q[4];        // Q[t = c][16g + 4x .. +3]
        f32x4 kt[4];       // K^T[16g... see below]: kt[mt] = K[4g .. 4g+3][i = 16(c/4) + 4mt + c%4]
        f32x4 vt;          // V[4g .. 4g+3][col]
        f32x4 eta4;        // step sizes of tokens 4g .. 4g+3 (prologue)
    };
    auto read_ops = [&](ChunkOps& o, const unsigned char* sl) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            o.k[x] = *reinterpret_cast<const f32x4*>(sl + kOffK + swz_row(c, 4 * g + x));
            if (!kMaps)
                o.q[x] = *reinterpret_cast<const f32x4*>(sl + kOffQ + swz_row(c, 4 * g + x));
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            o.kt[mt] = *reinterpret_cast<const f32x4*>(
                sl + kOffKt + swz_kt(16 * (c >> 2) + 4 * mt + (c & 3), g));
        o.vt = *reinterpret_cast<const f32x4*>(sl + kOffVt + swz_vt(col, g));
        if constexpr (kPro)
            o.eta4 = *reinterpret_cast<const f32x4*>(sl + kSlotBytes + 16 * g);
    };

    auto step = [&](const ChunkOps& o, int t0) {
        // R = -V + K W_J, St = K Q^T, Yt = W_J^T Q^T: 4 accumulators each over
        // k-steps ks = 4x + r (x = register group of the row segment)
        f32x4 R[4], St[4], Yt[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            R[r] = (r == 0) ? -o.vt : zero;
            St[r] = zero;
            Yt[r] = zero;
        }
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // k-step ks = 4x + r: i = 16g + ks, W operand Wacc[x][r]
                R[r] = mfma(o.k[x][r], Wacc[x][r], R[r]);
                if constexpr (!kMaps) {
                    St[r] = mfma(o.k[x][r], o.q[x][r], St[r]);
                    Yt[r] = mfma(Wacc[x][r], o.q[x][r], Yt[r]);
                }
            }
        const f32x4 Rs = (R[0] + R[1]) + (R[2] + R[3]);

        // E' = -eta R: lane (c = j, g) holds E'[t = 4g + q][j]
        const f32x4 Ep = kPro ? -(o.eta4 * Rs) : -et * Rs;

        // W += K^T E' (k-steps q over tokens t = 4g + q)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                Wacc[mt] = mfma(o.kt[mt][qq], Ep[qq], Wacc[mt]);

        if constexpr (!kMaps) {
            f32x4 S = (St[0] + St[1]) + (St[2] + St[3]);
            const f32x4 Ys = (Yt[0] + Yt[1]) + (Yt[2] + Yt[3]);
            // S^T masked: lane (c = t, g) holds S[t][t' = 4g + q]; keep t' <= t
            // (the chunk-start read drops the intra-chunk term)
            const bool keep = !(kPro && pro.read_start);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                S[qq] = (keep && 4 * g + qq <= c) ? S[qq] : 0.f;
            f32x4 Y2 = zero;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                Y2 = mfma(Ep[qq], S[qq], Y2);
            const f32x4 Yv = Ys + Y2;

            // Y[t0 + c][16w + 4g .. +3]; rows past the segment fall outside the buffer
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, Yv), ry,
                                                   ((t0 + c) * kD + 16 * w + 4 * g) * 4, 0, 0);
        }
    };

    auto process = [&](const StageRegs& next, int chunk, int slot, StageRegs& ahead) {
        write_stage(next, (slot + 1) % kSlots);
        __syncthreads();
        ChunkOps o;
        read_ops(o, lds + slot * kSlotB);
        step(o, chunk * kB);
        prep(ahead, chunk + 2);
    };

    if (nchunks > 0) {
        StageRegs setA[kSetK], setB[kSetK];
        {
            StageRegs first;
            load_stage(first, 0);
            prep(first, 0);
            write_stage(first, 0);
        }
#pragma unroll
        for (int p = 0; p < kSetK; ++p)
            load_stage(setA[p], 1 + p);
        prep(setA[0], 1);
        for (int c0 = 0; c0 < nchunks; c0 += 2 * kSetK) {
#pragma unroll
            for (int p = 0; p < kSetK; ++p)
                load_stage(setB[p], c0 + kSetK + 1 + p);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = 0; p < kSetK; ++p) {
                if (c0 + p >= nchunks)       // uniform: the scan is done
                    goto done;
                process(setA[p], c0 + p, p % kSlots, p + 1 < kSetK ? setA[p + 1] : setB[0]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = 0; p < kSetK; ++p)
                load_stage(setA[p], c0 + 2 * kSetK + 1 + p);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = 0; p < kSetK; ++p) {
                if (c0 + kSetK + p >= nchunks)
                    goto done;
                process(setB[p], c0 + kSetK + p, (kSetK + p) % kSlots,
                        p + 1 < kSetK ? setB[p + 1] : setA[0]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
done:

    float* wo;
    if (kMaps)
        wo = map_ptr(s) + half * kD * kD;
    else if (s == nseg - 1)
        wo = W_out + u * kD * kD;
    else
        return;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            wo[wrow(mt, 4 * g + r) * kD + col] = Wacc[mt][r];
}

}  // namespace

bool linear_mfma_f32_supports(const LinearArgs& a)
{
    const int64_t max_tokens = (int64_t{1} << 31) / (kD * 4) - kB * (3 * kSet + 2);
    return a.dtype == 0 && a.d == kD && a.b == kB && a.T <= max_tokens;
}

namespace {

template <bool kPro>
hipError_t launch_f32(const LinearArgs& a, const SegmentPlan& p)
{
    const auto* q = static_cast<const float*>(a.Q);
    const auto* k = static_cast<const float*>(a.K);
    const auto* v = static_cast<const float*>(a.V);
    auto* y = static_cast<float*>(a.Y);
    const int H = static_cast<int>(a.H), T = static_cast<int>(a.T);
    const int seg_len = static_cast<int>(p.seg_len);
    const int64_t units = a.B * a.H;
    const int lds = kSlots * (kPro ? kSlotBytes + kB * 4 : kSlotBytes);
    if (p.nseg > 1) {
        const dim3 grid(static_cast<unsigned>(placed_grid(units, 2 * (p.nseg - 1))));
        hipLaunchKernelGGL((linear_mfma_f32_kernel<true, kPro>), grid, dim3(kThreads), lds, a.stream, q,
                           k, v, a.W0, a.w0_per_batch, a.eta, H, T, units, seg_len, p.nseg, p.maps,
                           p.wstart, y, a.W_out, a.pro);
        hipError_t e = hipGetLastError();
        if (e == hipSuccess)
            e = launch_linear_combine(a, p);
        if (e != hipSuccess || p.starts_only)
            return e;
    }
    const dim3 grid(static_cast<unsigned>(p.nseg > 1 ? placed_grid(units, p.nseg) : units));
    hipLaunchKernelGGL((linear_mfma_f32_kernel<false, kPro>), grid, dim3(kThreads), lds, a.stream, q, k,
                       v, a.W0, a.w0_per_batch, a.eta, H, T, units, seg_len, p.nseg, p.maps, p.wstart,
                       y, a.W_out, a.pro);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_mfma_f32(const LinearArgs& a, const SegmentPlan& p)
{
    return a.pro.active() ? launch_f32<true>(a, p) : launch_f32<false>(a, p);
}

}  // namespace ttt
