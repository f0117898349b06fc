// ttt_momentum_mfma.hip -- the momentum scan of ttt_momentum.hip on MFMA for
// bf16 Q/K/V, d = 64, b = 16, fp32 W and M (the E2-TTT write-up on
// zhichai.net, sections "E2-TTT's Breakthrough" and "Core Math").
//
// Per chunk of n <= 16 tokens from (W, M), with the chunk closed form of
// ttt_momentum.hip (c_t = beta + .. + beta^t, dsum_m = 1 + .. + beta^m):
//   RHS = K W - V - eta diag(c_t) K M           (exact steps; K W - V else)
//   R   = P RHS,  P = (I + eta A)^-1            (exact steps; R = RHS else)
//   W  <- W - eta c_n M + K^T (-eta dsum_{n-1-t} R)
//   M  <- beta^n M + K^T (beta^{n-1-t} R)
//   Y   = Q W + (-eta c_{t+1} Q) M + (-eta S o Dsum) R
// P depends on the chunk's keys only (A[t][u] = dsum_{t-1-u} k_t . k_u,
// u < t), so a first launch computes every chunk's P at once, off the
// chain: one wave per 4 chunks, K K^T on MFMA, then each lane solves one row
// of P from P (I + eta A) = I in fp32 (a unit lower triangular system, 120
// fused multiply-adds per row).  P goes to the caller's workspace as bf16 in
// the A-operand layout of the scan, two chunks interleaved per lane, so that
// the scan loads it with one 16-byte load per lane per stage of two chunks.
//
// The scan: one workgroup (4 waves) per (batch, head) chain.  Every step of
// the recurrence acts on the output columns of W and M separately (the
// residual of column j needs only column j of W, M and V), so wave w owns
// columns [16w, 16w + 16) of both, as fp32 MFMA accumulators with rows in the
// rho order of ttt_mfma_ops.h: rounded to bf16 they are at once the B
// operand of K W, K M and the A operand of W^T Q^T, M^T Q^T.  R (C layout)
// rounded to bf16 is the B operand of the state updates K^T (.) and the A
// operand of R^T S^T.  K M and M^T Q^T come out in accumulators of their
// own, so that their row scalings by token (c_t, c_{t+1}) are four fused
// multiply-adds on the C tile rather than a rescaled operand; the geometric
// weights on R and the Dsum mask on S are per-lane constants too (lane (c, g)
// of a C tile holds tokens 4g .. 4g+3, of S^T and Y^T token c).
// Inputs are staged through a 3-slot LDS ring two chunks at a time, loaded 3
// to 6 stages ahead in two register sets, with one barrier per stage, as in
// the plain bf16 scan (ttt_linear_mfma.hip).  The loop runs the stages before
// the one holding the last token, all full; that last stage runs after it,
// each chunk with the update weights of its own token count (a chunk past the
// last token is skipped: with momentum an all-zero chunk still moves W).
//
// With beta = 0 for the chain's head, M plays no part in the recurrence: the
// chain runs a loop without the M products (for exact steps, the delta rule
// with its chunked triangular solve), and M_out is the last token's gradient.
#include "ttt_mfma_ops.h"

namespace ttt {
namespace {

using namespace mfma;

constexpr int kD = 64;
constexpr int kB = 16;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStageChunks = 2;
constexpr int kStageTokens = kB * kStageChunks;
constexpr int kSet = 3;                 // stages per register set (two sets)
constexpr int kSlots = 3;               // LDS ring slots
constexpr int kOffK = 0;
constexpr int kOffQ = kOffK + kB * kRowBytes;
constexpr int kOffV = kOffQ + kB * kRowBytes;
constexpr int kChunkBytes = kOffV + kB * kRowBytes;
constexpr int kSlotBytes = kChunkBytes * kStageChunks;
constexpr int kPinvStageBytes = 64 * 16;   // two chunks' P, 16 bytes per lane

static_assert((2 * kSet) % kSlots == 0, "slot index must be static inside the loop");

// sum_{s = lo}^{hi} beta^s (0 when hi < lo), lo and hi in [0, 16]
__device__ __forceinline__ float geo(float beta, int lo, int hi)
{
    float acc = 0.f, p = 1.f;
#pragma unroll
    for (int s = 0; s <= kB; ++s) {
        if (s >= lo && s <= hi)
            acc += p;
        p *= beta;
    }
    return acc;
}

// ---------------------------------------------------------------------------
// P = (I + eta A)^-1 of every chunk
// ---------------------------------------------------------------------------
constexpr int kInvChunksPerWave = 4;
constexpr int kInvWaves = 4;

__global__ void __launch_bounds__(64 * kInvWaves)
momentum_inverse_kernel(const uint16_t* __restrict__ K, const float* __restrict__ eta,
                        const float* __restrict__ beta, int H, int T, int nchunks, int nstages,
                        int64_t total, unsigned char* __restrict__ pinv)
{
    // eta A of each chunk, column-major: ncol[wave][chunk][u][t]
    __shared__ __attribute__((aligned(16))) float ncol[kInvWaves][kInvChunksPerWave][kB][kB];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int64_t first = (static_cast<int64_t>(blockIdx.x) * kInvWaves + w) * kInvChunksPerWave;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    for (int q = 0; q < kInvChunksPerWave; ++q) {
        const int64_t id = first + q;
        if (id >= total)                 // uniform over the wave
            break;
        const int64_t u = id / nchunks;
        const int ci = static_cast<int>(id - u * nchunks);
        const int h = static_cast<int>(u % H);
        const float et = eta[h], bt = beta[h];
        // lane (c, g): inputs 8g .. 8g+7 and 32 + 8g .. of token 16 ci + c
        const int t = ci * kB + c;
        u32x4 k0 = {0u, 0u, 0u, 0u}, k1 = {0u, 0u, 0u, 0u};
        if (t < T) {
            const uint16_t* row = K + (u * T + t) * kD;
            k0 = *reinterpret_cast<const u32x4*>(row + 8 * g);
            k1 = *reinterpret_cast<const u32x4*>(row + 32 + 8 * g);
        }
        const bf16x8 a0 = __builtin_bit_cast(bf16x8, k0), a1 = __builtin_bit_cast(bf16x8, k1);
        // K K^T: lane (c, g) receives (k_{4g+e} . k_c), e = 0..3
        f32x4 G = mfma32(a0, a0, zero);
        G = mfma32(a1, a1, G);
        f32x4 n4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tt = 4 * g + e;     // row t of A, column u = c
            n4[e] = c < tt ? et * geo(bt, 0, tt - 1 - c) * G[e] : 0.f;
        }
        *reinterpret_cast<f32x4*>(&ncol[w][q][c][4 * g]) = n4;
    }
    __syncthreads();

    // lane (q, t) = (l / 16, l % 16): row t of the q-th chunk's P, from
    // P (I + N) = I with N strictly lower: P[t][u] = (t == u) - sum_{v > u}
    // P[t][v] N[v][u], u from 15 down to 0 (rows above t come out zero)
    const int q = g, t = c;
    const int64_t id = first + q;
    if (id >= total)
        return;
    float pr[kB];
#pragma unroll
    for (int uu = kB - 1; uu >= 0; --uu) {
        const float* col = &ncol[w][q][uu][0];
        float acc = uu == t ? 1.f : 0.f;
#pragma unroll
        for (int v = uu + 1; v < kB; ++v)
            acc -= pr[v] * col[v];
        pr[uu] = acc;
    }
    // A operand of the scan: lane t + 16 gp holds P[t][4gp .. 4gp + 3]
    const int64_t u = id / nchunks;
    const int ci = static_cast<int>(id - u * nchunks);
    unsigned char* dst = pinv + (u * nstages + ci / 2) * kPinvStageBytes + (ci & 1) * 8;
#pragma unroll
    for (int gp = 0; gp < 4; ++gp) {
        const bf16x4 x = pack4(f32x4{pr[4 * gp], pr[4 * gp + 1], pr[4 * gp + 2], pr[4 * gp + 3]});
        *reinterpret_cast<u32x2*>(dst + (t + 16 * gp) * 16) = __builtin_bit_cast(u32x2, x);
    }
}

// ---------------------------------------------------------------------------
// the scan
// ---------------------------------------------------------------------------
struct ScanParams {
    const uint16_t* Q; const uint16_t* K; const uint16_t* V;
    const float* W0; int w0_per_batch; const float* M0;
    const float* eta; const float* beta; int H; int T;
    const unsigned char* pinv;
    uint16_t* Y; float* W_out; float* M_out;
    int64_t units;
    // sequence segments: nseg of seg_len tokens (a multiple of a stage; the
    // last one shorter), the maps of segments 0 .. nseg - 2 and the start
    // states [W; M] of every segment ([units][nseg][2][d][d])
    int nseg; int seg_len;
    float* maps; const float* xstart;
};

// a segment's map: A (2d x 2d, acting on a column [W; M] of the state), then
// N (2d x d), row-major
constexpr int64_t kMapFloats = 4 * kD * kD + 2 * kD * kD;

// update weights of a chunk of n tokens, for this lane's C-tile rows
// t = 4g + e: W gets -eta dsum_{n-1-t} R[t], M gets beta^{n-1-t} R[t]; the
// chunk-start M enters W with -eta c_n and M with beta^n
struct Coef {
    f32x4 ud, um;
    float wm, mm;
};

__device__ __forceinline__ Coef chunk_coef(float et, float bt, int n, int g)
{
    Coef cf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = 4 * g + e;
        const int m = n - 1 - t;
        cf.ud[e] = t < n ? -et * geo(bt, 0, m) : 0.f;
        cf.um[e] = t < n ? geo(bt, m, m) : 0.f;
    }
    cf.wm = -et * geo(bt, 1, n);
    cf.mm = geo(bt, n, n);
    return cf;
}

// One chain, or one segment `seg` of it.  kMap: the segment's affine map
// instead of its outputs.  A segment maps each column [W; M] of the state to
// A [W; M] + n (the recurrence treats the d columns alike, n from column j
// of V), so the map is the segment run on 3d columns with no readout: part 0
// starts from W = e_j, M = 0 and part 1 from W = 0, M = e_j with V = 0 (the
// columns of A), part 2 from zero with V (N).
template <bool kExact, bool kMom, bool kMap>
__device__ __forceinline__ void scan_chain(const ScanParams& p, unsigned char* lds, int64_t u,
                                           int h, int seg, int part)
{
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int col = 16 * w + c;
    // the segment's tokens [t_begin, t_begin + T) of the chain
    const int64_t t_begin = static_cast<int64_t>(seg) * p.seg_len;
    const int T = p.nseg > 1 ? static_cast<int>(min(static_cast<int64_t>(p.seg_len), p.T - t_begin))
                             : p.T;
    const float et = p.eta[h];
    const float bt = kMom ? p.beta[h] : 0.f;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // W and M: acc[mt][r] = X[rho(mt, 4g + r)][col]
    f32x4 Wacc[4], Macc[4];
    if constexpr (kMap) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = rho(mt, 4 * g + r) == col ? 1.f : 0.f;
                Wacc[mt][r] = part == 0 ? e : 0.f;
                Macc[mt][r] = part == 1 ? e : 0.f;
            }
    } else {
        const float* w0 = p.W0 + (p.w0_per_batch ? u : h) * kD * kD;
        const float* m0 = p.M0 ? p.M0 + u * kD * kD : nullptr;
        if (p.nseg > 1) {
            w0 = p.xstart + (u * p.nseg + seg) * 2 * kD * kD;
            m0 = w0 + kD * kD;
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                Wacc[mt][r] = w0[rho(mt, 4 * g + r) * kD + col];
                Macc[mt][r] = m0 ? m0[rho(mt, 4 * g + r) * kD + col] : 0.f;
            }
    }

    // -I as the B operand of a 16x16x16 product: B[k = 4g + r][n = c] = -(k == n)
    bf16x4 neg_eye;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        neg_eye[r] = static_cast<__bf16>(4 * g + r == c ? -1.0f : 0.0f);

    // per-lane scalings: the K M rows of the residual (C layout, tokens
    // 4g + e), the q M readout (token c), and S^T (lane (c, g) holds
    // S[c][4g + e]) masked to u <= t and weighted -eta dsum_{t-u}
    f32x4 kc4;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        kc4[e] = -et * geo(bt, 1, 4 * g + e);
    const float qc = -et * geo(bt, 1, c + 1);
    f32x4 sc;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int uu = 4 * g + e;
        sc[e] = uu <= c ? -et * geo(bt, 0, c - uu) : 0.f;
    }
    const Coef full = chunk_coef(et, bt, kB, g);
    const Coef tail = chunk_coef(et, bt, T % kB, g);

    const int64_t base = (u * static_cast<int64_t>(p.T) + t_begin) * kD;
    const int64_t bytes = static_cast<int64_t>(T) * kD * 2;
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(p.Q + base, bytes);
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(p.K + base, bytes);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(p.V + base, bytes);
    const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(p.Y + base, bytes);
    const int nstages = (T + kStageTokens - 1) / kStageTokens;
    // the chain's P, from the segment's first stage on
    const int64_t pstage = u * ((p.T + kStageTokens - 1) / kStageTokens) + t_begin / kStageTokens;
    const __amdgpu_buffer_rsrc_t rp =
        buffer_rsrc(kExact ? p.pinv + pstage * kPinvStageBytes : p.pinv,
                    kExact ? static_cast<int64_t>(nstages) * kPinvStageBytes : 0);

    struct StageRegs {
        u32x4 k, q, v, pv;
    };
    const int st_row = 8 * w + (lane >> 3);             // 0..31
    const int st_seg = lane & 7;
    auto load_stage = [&](StageRegs& o, int stage) {
        const int off = (stage * kStageTokens + st_row) * kRowBytes + st_seg * 16;
        o.k = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        if constexpr (!kMap)
            o.q = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
        o.v = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
        if (kExact)
            o.pv = __builtin_amdgcn_raw_buffer_load_b128(rp, stage * kPinvStageBytes + lane * 16, 0, 0);
    };
    auto write_stage = [&](const StageRegs& o, int slot) {
        unsigned char* chunk = lds + slot * kSlotBytes + (st_row >> 4) * kChunkBytes;
        const int r = st_row & 15;
        *reinterpret_cast<u32x4*>(chunk + kOffK + swz(r, st_seg)) = o.k;
        if constexpr (!kMap)
            *reinterpret_cast<u32x4*>(chunk + kOffQ + swz(r, st_seg)) = o.q;
        *reinterpret_cast<u32x4*>(chunk + kOffV + swz(r, st_seg)) = o.v;
    };

    struct ChunkOps {
        bf16x8 ka0, ka1, qa0, qa1;
        bf16x4 vrow;
        bf16x4 kt[4];
    };
    auto read_ops = [&](ChunkOps& o, const unsigned char* tile) {
        o.ka0 = *reinterpret_cast<const bf16x8*>(tile + kOffK + swz(c, g));
        o.ka1 = *reinterpret_cast<const bf16x8*>(tile + kOffK + swz(c, 4 + g));
        if constexpr (!kMap) {
            o.qa0 = *reinterpret_cast<const bf16x8*>(tile + kOffQ + swz(c, g));
            o.qa1 = *reinterpret_cast<const bf16x8*>(tile + kOffQ + swz(c, 4 + g));
        }
        // the columns of A run with V = 0
        if (!kMap || part == 2)
            o.vrow = *reinterpret_cast<const bf16x4*>(tile + kOffV + swz(c, 2 * w + (g >> 1)) + 8 * (g & 1));
        else
            o.vrow = bf16x4{};
        // K^T (A operand of the updates), transposed on the way out of LDS:
        // lane (c, g) receives K[4g + r][rho(mt, c)], r = 0..3
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            o.kt[mt] = read_tr16(tile + kOffK + swz(4 * g + (c >> 2), 4 * (mt >> 1) + (c & 3)) + 8 * (mt & 1));
    };

    // One chunk, tokens t0 .. t0 + n - 1 (n given through cf); pa: this
    // lane's A-operand piece of the chunk's P; last: the chunk holds token T-1.
    auto step = [&](const ChunkOps& o, bf16x4 pa, int t0, const Coef& cf, bool last) {
        const bf16x8 wb0 = pack8(Wacc[0], Wacc[1]);
        const bf16x8 wb1 = pack8(Wacc[2], Wacc[3]);
        bf16x8 mb0, mb1;
        if constexpr (kMom) {
            mb0 = pack8(Macc[0], Macc[1]);
            mb1 = pack8(Macc[2], Macc[3]);
        }
        // RHS = K W - V (- eta diag(c_t) K M), C layout: rows t = 4g + r, column col
        f32x4 R = mfma16_as32(o.vrow, neg_eye, zero);
        R = mfma32(o.ka0, wb0, R);
        R = mfma32(o.ka1, wb1, R);
        if constexpr (kExact && kMom) {
            f32x4 KM = mfma32(o.ka0, mb0, zero);
            KM = mfma32(o.ka1, mb1, KM);
            R += kc4 * KM;
        }
        if constexpr (kExact)
            R = mfma16(pa, pack4(R), zero);        // R = P RHS

        // state updates; the chunk-start M enters before R is known
        const bf16x4 ew = pack4(cf.ud * R);
        if constexpr (kMom) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                Wacc[mt] = mfma16(o.kt[mt], ew, Wacc[mt] + cf.wm * Macc[mt]);
            const bf16x4 em = pack4(cf.um * R);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                Macc[mt] = mfma16(o.kt[mt], em, cf.mm * Macc[mt]);
        } else {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                Wacc[mt] = mfma16(o.kt[mt], ew, Wacc[mt]);
            if (last) {        // beta = 0: M is the last token's gradient
                const bf16x4 em = pack4(cf.um * R);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    Macc[mt] = mfma16(o.kt[mt], em, zero);
            }
        }

        if constexpr (kMap)
            return;
        // off the chain: Y^T = W^T Q^T (+ M^T (-eta c_{t+1} Q)^T) + R^T S~^T
        f32x4 St = mfma32(o.ka0, o.qa0, zero);
        St = mfma32(o.ka1, o.qa1, St);
        f32x4 Yt = mfma32(wb0, o.qa0, zero);
        Yt = mfma32(wb1, o.qa1, Yt);
        Yt = mfma16_as32(pack4(R), pack4(sc * St), Yt);
        if constexpr (kMom) {
            // lane (c, g) holds token c: (q_c M)[4g + r] scaled by -eta c_{c+1}
            f32x4 Ym = mfma32(mb0, o.qa0, zero);
            Ym = mfma32(mb1, o.qa1, Ym);
            Yt += qc * Ym;
        }
        // Y[t0 + c][16w + 4g .. +3]; rows past the sequence fall outside the buffer
        const bf16x4 yb = pack4(Yt);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, yb), ry,
                                              ((t0 + c) * kD + 16 * w + 4 * g) * 2, 0, 0);
    };

    u32x4 pcur = {0u, 0u, 0u, 0u};      // P of the stage being computed
    // Stage s (two full chunks, before the stage of the last token):
    // publish stage s + 1 (held in `next`), then compute stage s.
    auto process = [&](const StageRegs& next, int s, int slot) {
        write_stage(next, (slot + 1) % kSlots);
        __syncthreads();
        const unsigned char* sl = lds + slot * kSlotBytes;
        const bf16x4 p0 = __builtin_bit_cast(bf16x4, u32x2{pcur[0], pcur[1]});
        const bf16x4 p1 = __builtin_bit_cast(bf16x4, u32x2{pcur[2], pcur[3]});
        if (kExact)
            pcur = next.pv;
        const int t0 = s * kStageTokens;
        ChunkOps o0, o1;
        read_ops(o0, sl);
        read_ops(o1, sl + kChunkBytes);
        step(o0, p0, t0, full, false);
        step(o1, p1, t0 + kB, full, false);
    };
    // the stages before the one holding token T - 1 run in the loop
    const int nloop = nstages - 1;

    if (nstages > 0) {
        StageRegs setA[kSet], setB[kSet];
        {
            StageRegs first;
            load_stage(first, 0);
            write_stage(first, 0);
            if (kExact)
                pcur = first.pv;
        }
#pragma unroll
        for (int q = 0; q < kSet; ++q)
            load_stage(setA[q], 1 + q);
        // stages s0 .. s0 + 2 kSet - 1 per iteration; setA holds s0 + 1 .. s0 + kSet
        for (int s0 = 0; s0 < nstages; s0 += 2 * kSet) {
#pragma unroll
            for (int q = 0; q < kSet; ++q)
                load_stage(setB[q], s0 + kSet + 1 + q);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < kSet; ++q) {
                if (s0 + q >= nloop)         // uniform: only the last stage is left
                    goto last;
                process(setA[q], s0 + q, q % kSlots);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < kSet; ++q)
                load_stage(setA[q], s0 + 2 * kSet + 1 + q);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < kSet; ++q) {
                if (s0 + kSet + q >= nloop)
                    goto last;
                process(setB[q], s0 + kSet + q, (kSet + q) % kSlots);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    last:
        // the stage of token T - 1, already in its slot (written before the
        // previous stage's barrier, or before the loop); its chunks take the
        // update weights of their own token counts
        __syncthreads();
        const int s = nstages - 1;
        const unsigned char* sl = lds + (s % kSlots) * kSlotBytes;
        const bf16x4 p0 = __builtin_bit_cast(bf16x4, u32x2{pcur[0], pcur[1]});
        const bf16x4 p1 = __builtin_bit_cast(bf16x4, u32x2{pcur[2], pcur[3]});
        const int t0 = s * kStageTokens;
        ChunkOps o0;
        read_ops(o0, sl);
        step(o0, p0, t0, t0 + kB <= T ? full : tail, t0 + kB >= T);
        if (t0 + kB < T) {
            ChunkOps o1;
            read_ops(o1, sl + kChunkBytes);
            step(o1, p1, t0 + kB, t0 + 2 * kB <= T ? full : tail, true);
        }
    }
    if constexpr (kMap) {
        // A[i][64 part + col] (part 0, 1) or N[i][col] (part 2), rows i of
        // W, then of M
        float* m = p.maps + (u * (p.nseg - 1) + seg) * kMapFloats;
        const int ld = part < 2 ? 2 * kD : kD;
        float* dst = part < 2 ? m + kD * part + col : m + 4 * kD * kD + col;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dst[rho(mt, 4 * g + r) * ld] = Wacc[mt][r];
                dst[(kD + rho(mt, 4 * g + r)) * ld] = Macc[mt][r];
            }
    } else if (seg == p.nseg - 1) {
        float* wo = p.W_out + u * kD * kD;
        float* mo = p.M_out + u * kD * kD;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                wo[rho(mt, 4 * g + r) * kD + col] = Wacc[mt][r];
                mo[rho(mt, 4 * g + r) * kD + col] = Macc[mt][r];
            }
    }
}

// kMap: the maps of segments 0 .. nseg - 2 (three workgroups per segment,
// see scan_chain); else the scans of the chains or of their segments.  With
// segments, the workgroups of a chain share an XCD (xcd_block).
template <bool kExact, bool kMap>
__global__ void __launch_bounds__(kThreads, 1)
momentum_mfma_kernel(ScanParams p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    int64_t u = blockIdx.x;
    int s = 0;
    if (p.nseg > 1) {
        xcd_block(static_cast<int>(blockIdx.x), kMap ? 3 * (p.nseg - 1) : p.nseg, p.units, u, s);
        if (u >= p.units)                // uniform over the workgroup
            return;
    }
    const int h = static_cast<int>(u % p.H);
    if constexpr (kMap)
        scan_chain<kExact, true, true>(p, lds, u, h, s / 3, s % 3);
    else if (p.beta[h] != 0.f)
        scan_chain<kExact, true, false>(p, lds, u, h, s, 0);
    else
        scan_chain<kExact, false, false>(p, lds, u, h, s, 0);
}

int64_t pinv_stages(int64_t T) { return (T + kStageTokens - 1) / kStageTokens; }

}  // namespace

bool momentum_mfma_supports(const MomentumArgs& a)
{
    // per-chain byte offsets, including the loads past the end, are 32-bit
    const int64_t max_tokens = (int64_t{1} << 31) / (kD * 2) - kStageTokens * (2 * kSet + 2);
    return a.dtype == 1 && a.d == kD && a.b == kB && a.T <= max_tokens;
}

namespace {

int64_t pad256(int64_t n) { return (n + 255) / 256 * 256; }

int64_t pinv_bytes(const MomentumArgs& a)
{
    return a.grad_mode == 0 ? pad256(a.B * a.H * pinv_stages(a.T) * kPinvStageBytes) : 0;
}

}  // namespace

// The chunk inverses (exact steps), then with nseg > 1 segments the maps of
// segments 0 .. nseg - 2 and the start states of all of them.
int64_t momentum_mfma_workspace_bytes(const MomentumArgs& a, int nseg)
{
    const int64_t units = a.B * a.H;
    int64_t n = pinv_bytes(a);
    if (nseg > 1)
        n += pad256(units * (nseg - 1) * kMapFloats * 4) + units * nseg * 2 * kD * kD * 4;
    return n;
}

// nseg segments of seg_len tokens (a multiple of a stage of two chunks, so
// that each segment's chunk inverses start at a stage of the chain's).
hipError_t launch_momentum_mfma(const MomentumArgs& a, void* workspace, int nseg, int64_t seg_len)
{
    const int64_t units = a.B * a.H;
    const bool exact = a.grad_mode == 0;
    auto* pinv = static_cast<unsigned char*>(workspace);
    const int T = static_cast<int>(a.T);
    if (T == 0 || nseg < 1 || (nseg > 1 && (seg_len % kStageTokens != 0 || seg_len * (nseg - 1) >= T)))
        nseg = 1;
    if (exact && T > 0) {
        const int nchunks = (T + kB - 1) / kB;
        const int64_t total = units * nchunks;
        const int64_t per_block = kInvWaves * kInvChunksPerWave;
        const dim3 grid(static_cast<unsigned>((total + per_block - 1) / per_block));
        hipLaunchKernelGGL(momentum_inverse_kernel, grid, dim3(64 * kInvWaves), 0, a.stream,
                           static_cast<const uint16_t*>(a.K), a.eta, a.beta,
                           static_cast<int>(a.H), T, nchunks, static_cast<int>(pinv_stages(T)),
                           total, pinv);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    float* maps = nullptr;
    float* xstart = nullptr;
    if (nseg > 1) {
        maps = reinterpret_cast<float*>(pinv + pinv_bytes(a));
        xstart = maps + pad256(units * (nseg - 1) * kMapFloats * 4) / 4;
    }
    ScanParams p{static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                 static_cast<const uint16_t*>(a.V), a.W0, a.w0_per_batch, a.M0, a.eta, a.beta,
                 static_cast<int>(a.H), T, pinv, static_cast<uint16_t*>(a.Y), a.W_out, a.M_out,
                 units, nseg, static_cast<int>(nseg > 1 ? seg_len : T), maps, xstart};
    const int lds = kSlots * kSlotBytes;
    if (nseg > 1) {
        const dim3 grid(static_cast<unsigned>(placed_grid(units, 3 * (nseg - 1))));
        if (exact)
            hipLaunchKernelGGL((momentum_mfma_kernel<true, true>), grid, dim3(kThreads), lds, a.stream, p);
        else
            hipLaunchKernelGGL((momentum_mfma_kernel<false, true>), grid, dim3(kThreads), lds, a.stream, p);
        hipError_t e = hipGetLastError();
        if (e == hipSuccess)
            e = launch_momentum_combine(a, maps, nseg, xstart);
        if (e != hipSuccess)
            return e;
    }
    const dim3 grid(static_cast<unsigned>(nseg > 1 ? placed_grid(units, nseg) : units));
    if (exact)
        hipLaunchKernelGGL((momentum_mfma_kernel<true, false>), grid, dim3(kThreads), lds, a.stream, p);
    else
        hipLaunchKernelGGL((momentum_mfma_kernel<false, false>), grid, dim3(kThreads), lds, a.stream, p);
    return hipGetLastError();
}

}  // namespace ttt
