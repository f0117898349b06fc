// ttt_linear_cols_f32.hip -- TTT-Linear dual-form scan for fp32 Q/K/V (head
// dim d = 64, mini-batch b = 16) with each chain's fast weights split by
// columns over four workgroups.
//
// Every product of the dual form keeps the output columns of W apart:
//     E = K W - V,   Y = Q W - eta tril(Q K^T) E,   W' = W - eta K^T E
// column j of E, Y and W' needs only column j of W (and all of K, Q, column
// j of V) -- the inner loss separates over output columns ("Test-Time
// Training Layers: How Inner-Loop Gradient Descent Replaces the Transformer KV
// Cache ...", sections "The Core Mechanism" and "Hardware Parallelization").
// One (batch, head) chain therefore runs on four CUs, workgroup J owning the
// 16 columns [16J, 16J + 16).  That divides the fp32 MFMA work of a chunk
// -- the bound of the one-workgroup kernel in ttt_linear_mfma_f32.hip -- by
// four per CU, which is what a chain's sequential chunks need when there are
// few chains.
//
// Inside a workgroup the 64-row contraction is split over the 4 waves: wave
// w holds rows [16w, 16w + 16) of the slice in one accumulator tile (lane
// (c, g): rows 16w + 4g + r, column c) and forms the partial products of
// those rows,
//     P_w = K[:, 16w..] W_w,   R_w = Q[:, 16w..] W_w,   S_w^T = K[:, 16w..] Q[:, 16w..]^T,
// 4 k-steps of v_mfma_f32_16x16x4_f32 each (k-slot g of k-step r <-> input
// index 16w + 4g + r, so the W operand is the accumulator register r itself).
// The partial tiles go to LDS in the accumulator's lane order; after the
// chunk's one barrier every wave adds the four P tiles in the same order
// (E = sum P - V, identical in every wave) and updates its rows,
//     W_w += K[:, 16w..]^T (-eta E)     (4 k-steps over the 16 tokens),
// and adds the R and S^T tiles too, forming
//     Y = R - eta tril(S) E             (S^T read as an A operand is S),
// of which wave w stores row 4g + w of each lane group: every wave does the
// same work, so no wave holds up the next barrier, and no memory operation
// sits under a branch (which would cost the loads' wait counts their
// precision: the stage loads of the chunks ahead must stay in flight).
// Partial tiles alternate between two LDS buffers by chunk parity, and the
// chunk tiles (K, Q, the V column slice) sit in a 3-slot LDS ring written two
// chunks ahead from a ring of 4 register sets loaded 6 chunks ahead, so one
// barrier per chunk orders everything.
//
// kMaps = true computes the affine map W_end = M W_start + N of a segment
// (half 0: from W = I with V = 0, giving M; half 1: from W = 0, giving N),
// column slice J of each, as the segment scan needs (see ttt_internal.h); the
// workgroups of segment 0 also copy W0 into the workspace.  The scan of
// segment s then composes its own start state from that copy,
//     W_{j+1} = M_j W_j + N_j,   j = 0 .. s - 1,
// in the same layout (each step: the waves' row tiles to LDS, transposed,
// one barrier, 16 k-steps over the 64 rows), so the start states need no
// launch of their own and never go through memory; segment s is ready after
// s steps, the last one after nseg - 1, as with a separate composition.
#include "ttt_mfma_ops.h"

namespace ttt {
namespace {

constexpr int kD = 64;
constexpr int kB = 16;
constexpr int kSlices = 4;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRing = 4;                         // register sets of staged chunks
constexpr int kSlots = 3;                        // LDS tile slots
constexpr int kP = kD + 4;                       // padded K, Q row (floats)
constexpr int kVP = 20;                          // padded V slice row (floats)
constexpr int kTileFloats = 256;                 
// LDS layout (floats): a slot holds the chunk's K, Q (scan only) and V slice
// (and with the prologue its 16 step sizes); the partial tiles [2 parity]
// [kinds][4 waves][256] follow the slots (the maps have only P, and no Q:
// 25 KB, so several share a CU)
template <bool kMaps, bool kPro>
struct Lay {
    static constexpr int kOffK = 0;
    static constexpr int kOffQ = kOffK + kB * kP;
    static constexpr int kOffV = kOffQ + (kMaps ? 0 : kB * kP);
    static constexpr int kOffEta = kOffV + kB * kVP;
    static constexpr int kSlotFloats = kOffEta + (kPro ? kB : 0);
    static constexpr int kKinds = kMaps ? 1 : 3;
    static constexpr int kOffPart = kSlots * kSlotFloats;
    static constexpr int kFloats = kOffPart + 2 * kKinds * kWaves * kTileFloats;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct StageRegs {
    u32x4 k, q, v;     // 16 bytes of K and Q row tid / 16; of the V slice (tid < 64)
    uint32_t eta;      // step size of row tid / 16 (prologue, per-token step sizes)
};

// kPro: the input prologue (Prologue in ttt_internal.h) applied as a chunk is
// written to LDS: its K and Q rows LayerNorm'd over the head dim (16 lanes
// per row, DPP sums) and its step sizes beside the tiles, which scale the
// residual rows, E'[t] = -eta_t E[t]; with read_start the tril term is
// dropped (every token reads the chunk-start W).  The scan with the prologue
// runs 8 waves: waves 0-3 compute as above, waves 4-7 only stage (load,
// LayerNorm and write each chunk to LDS two chunks ahead, one barrier per
// chunk like the compute waves), so the normalisation's VALU work runs beside
// the chunk chain on the same SIMDs instead of inside it.
template <bool kMaps, bool kPro>
__global__ void __launch_bounds__(kPro && !kMaps ? 2 * kThreads : kThreads, 1)
linear_cols_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                       const float* __restrict__ V, const float* W0, int w0_per_batch,
                       const float* __restrict__ eta, int H, int T, int64_t units, int seg_len,
                       int nseg, float* maps, float* wstart, float* __restrict__ Y,
                       float* W_out, int compose, Prologue pro)
{
    using L = Lay<kMaps, kPro>;
    constexpr int kOffK = L::kOffK, kOffQ = L::kOffQ, kOffV = L::kOffV, kSlotFloats = L::kSlotFloats;
    __shared__ __attribute__((aligned(16))) float lds[L::kFloats];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int c = lane & 15;
    const int g = lane >> 4;
    constexpr bool kSplit = kPro && !kMaps;
    const bool stager = kSplit && w >= kWaves;   // waves 4-7 of the split scan
    const int sid = tid & (kThreads - 1);        // staging thread index

    // chain u, segment s (and map half), column slice J
    int64_t u;
    int sb;
    xcd_block(blockIdx.x, kMaps ? 2 * kSlices * (nseg - 1) : kSlices * nseg, units, u, sb);
    if (u >= units)                      // padding of the XCD placement
        return;
    const int J = sb % kSlices;
    const int half = kMaps ? (sb / kSlices) & 1 : 0;
    const int s = kMaps ? sb / (2 * kSlices) : sb / kSlices;
    const int h = static_cast<int>(u % H);
    const float et = eta[h];
    const int t_begin = s * seg_len;
    const int t_len = min(seg_len, T - t_begin);
    const int nchunks = (t_len + kB - 1) / kB;

    // Wr = rows 16w + 4g + r, column 16J + c of the slice
    f32x4 Wr;
    if (kMaps) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Wr[r] = (half == 0 && 16 * w + 4 * g + r == 16 * J + c) ? 1.f : 0.f;
    } else if (!stager) {
        const float* w0 = nseg > 1 ? wstart + (u * nseg + (compose ? 0 : s)) * kD * kD
                                   : W0 + (w0_per_batch ? u : h) * kD * kD;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Wr[r] = w0[(16 * w + 4 * g + r) * kD + 16 * J + c];
    }
    if (kMaps && s == 0 && half == 0) {
        // the copy of W0 the scans start from (W_out may overwrite W0)
        const float* w0 = W0 + (w0_per_batch ? u : h) * kD * kD;
        float* dst = wstart + u * nseg * kD * kD;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = (tid >> 4) + 16 * q;
            dst[i * kD + 16 * J + (tid & 15)] = w0[i * kD + 16 * J + (tid & 15)];
        }
    }
    if (!kMaps && compose && s > 0 && stager) {
        for (int j = 0; j <= s; ++j)     // the composition's s barriers and the one after it
            __syncthreads();
    } else if (!kMaps && compose && s > 0) {
        // W_s from W_0 through the maps of segments 0 .. s - 1; wave w's A
        // operand of k-step ks is M_j[16w + c][16g + ks] (a 64-byte run per
        // lane), its B operand W_j[16g + ks][c] from the transposed slice
        // [column][row] in LDS (two buffers by step parity); operands of step
        // j + kDepth load while step j runs
        constexpr int kDepth = 3;
        constexpr int kColP = kD + 4;            // [16 columns][kColP] per buffer
        f32x4 ma[kDepth][4], mn[kDepth];
        auto load_map = [&](f32x4 (&a)[4], f32x4& n, int j) {
            const float* M = maps + (u * (nseg - 1) + min(j, s - 1)) * 2 * kD * kD;
            const float* N = M + kD * kD;
#pragma unroll
            for (int x = 0; x < 4; ++x)
                a[x] = *reinterpret_cast<const f32x4*>(M + (16 * w + c) * kD + 16 * g + 4 * x);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                n[r] = N[(16 * w + 4 * g + r) * kD + 16 * J + c];
        };
#pragma unroll
        for (int q = 0; q < kDepth; ++q)
            load_map(ma[q], mn[q], q);
        auto cstep = [&](int q, int j) {
            float* Wt = lds + (j & 1) * 16 * kColP;
            *reinterpret_cast<f32x4*>(Wt + c * kColP + 16 * w + 4 * g) = Wr;
            __syncthreads();
            f32x4 b[4];
#pragma unroll
            for (int x = 0; x < 4; ++x)
                b[x] = *reinterpret_cast<const f32x4*>(Wt + c * kColP + 16 * g + 4 * x);
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            f32x4 acc[4] = {mn[q], zero, zero, zero};
#pragma unroll
            for (int ks = 0; ks < 16; ++ks)
                acc[ks & 3] = mfma(ma[q][ks >> 2][ks & 3], b[ks >> 2][ks & 3], acc[ks & 3]);
            Wr = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            load_map(ma[q], mn[q], j + kDepth);
        };
        int j0 = 0;
        for (; j0 + kDepth <= s; j0 += kDepth) {
#pragma unroll
            for (int q = 0; q < kDepth; ++q)
                cstep(q, j0 + q);
        }
#pragma unroll
        for (int q = 0; q < kDepth; ++q) {
            if (j0 + q >= s)             // uniform
                break;
            cstep(q, j0 + q);
        }
        __syncthreads();                 // the slice buffers are the tile slots below
    }

    const int64_t base = (u * static_cast<int64_t>(T) + t_begin) * kD;
    const int64_t seg_bytes = static_cast<int64_t>(t_len) * kD * 4;
    const __amdgpu_buffer_rsrc_t rq = mfma::buffer_rsrc(Q + base, kMaps ? 0 : seg_bytes);
    const __amdgpu_buffer_rsrc_t rk = mfma::buffer_rsrc(K + base, seg_bytes);
    const __amdgpu_buffer_rsrc_t rv = mfma::buffer_rsrc(V + base, (kMaps && half == 0) ? 0 : seg_bytes);
    const __amdgpu_buffer_rsrc_t ry = mfma::buffer_rsrc(Y + base, kMaps ? 0 : seg_bytes);

    // staging: thread tid moves 16 bytes of row tid / 16 of K and Q (columns
    // 4 (tid % 16) ..), and lane l of every wave loads 16 bytes of the V slice
    // (row l / 4, columns 16J + 4 (l % 4) ..), which wave 0 writes to LDS;
    // out-of-range reads give zeros
    const int st_row = sid >> 4;
    const int st_col = 4 * (sid & 15);
    const int sv_row = (sid & 63) >> 2;
    const int sv_col = 4 * (sid & 3);
    // prologue: gamma, beta of this thread's 4 columns
    const bool use_tok = kPro && pro.eta_tok != nullptr;
    const bool ln_k = kPro && pro.ln_k != nullptr;
    const bool ln_q = kPro && !kMaps && pro.ln_q != nullptr;
    float gk[4], bk[4], gq[4], bq[4];
    if constexpr (kPro) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            gk[e] = ln_k ? pro.ln_k[(2 * h) * kD + st_col + e] : 1.f;
            bk[e] = ln_k ? pro.ln_k[(2 * h + 1) * kD + st_col + e] : 0.f;
            gq[e] = ln_q ? pro.ln_q[(2 * h) * kD + st_col + e] : 1.f;
            bq[e] = ln_q ? pro.ln_q[(2 * h + 1) * kD + st_col + e] : 0.f;
        }
    }
    const __amdgpu_buffer_rsrc_t reta =
        mfma::buffer_rsrc(use_tok ? pro.eta_tok + u * static_cast<int64_t>(T) + t_begin : eta,
                   use_tok ? static_cast<int64_t>(t_len) * 4 : 0);
    auto load_stage = [&](StageRegs& o, int chunk) {
        const int off = ((chunk * kB + st_row) * kD + st_col) * 4;
        o.k = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        if (!kMaps)
            o.q = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
        o.v = __builtin_amdgcn_raw_buffer_load_b128(
            rv, ((chunk * kB + sv_row) * kD + 16 * J + sv_col) * 4, 0, 0);
        if (use_tok)
            o.eta = __builtin_amdgcn_raw_buffer_load_b32(reta, (chunk * kB + st_row) * 4, 0, 0);
    };
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
    auto write_stage = [&](const StageRegs& o, int chunk) {
        float* sl = lds + (chunk % kSlots) * kSlotFloats;
        u32x4 kx = o.k, qx = o.q;
        if constexpr (kPro) {
            const bool valid = chunk * kB + st_row < t_len;
            if (ln_k)
                kx = norm(kx, gk, bk, valid);
            if (ln_q)
                qx = norm(qx, gq, bq, valid);
            // (the 16 lanes of a row store the same value: no lane branch)
            sl[L::kOffEta + st_row] = use_tok ? __uint_as_float(o.eta) : et;
        }
        *reinterpret_cast<u32x4*>(sl + kOffK + st_row * kP + st_col) = kx;
        if (!kMaps)
            *reinterpret_cast<u32x4*>(sl + kOffQ + st_row * kP + st_col) = qx;
        if ((sid >> 6) == 0)
            *reinterpret_cast<u32x4*>(sl + kOffV + sv_row * kVP + sv_col) = o.v;
    };
    // partial tile `kind` (0 P, 1 R, 2 S^T) of wave wv, chunk parity par
    auto part = [&](int par, int kind, int wv) {
        return lds + L::kOffPart + ((par * L::kKinds + kind) * kWaves + wv) * kTileFloats + 4 * lane;
    };

    // one chunk: phase 1 (partials), the barrier, phase 2 (E, the update of
    // this wave's rows, Y)
    auto chunk_step = [&](int ch) {
        const float* sl = lds + (ch % kSlots) * kSlotFloats;
        const int par = ch & 1;
        const f32x4 krow = *reinterpret_cast<const f32x4*>(sl + kOffK + c * kP + 16 * w + 4 * g);
        f32x4 kt, vv;                    // K[4g + r][16w + c], V[4g + r][16J + c]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            kt[r] = sl[kOffK + (4 * g + r) * kP + 16 * w + c];
            vv[r] = sl[kOffV + (4 * g + r) * kVP + c];
        }
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 P = zero;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            P = mfma(krow[r], Wr[r], P);
        *reinterpret_cast<f32x4*>(part(par, 0, w)) = P;
        if (!kMaps) {
            const f32x4 qrow = *reinterpret_cast<const f32x4*>(sl + kOffQ + c * kP + 16 * w + 4 * g);
            f32x4 R = zero, St = zero;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                R = mfma(qrow[r], Wr[r], R);
                St = mfma(krow[r], qrow[r], St);
            }
            *reinterpret_cast<f32x4*>(part(par, 1, w)) = R;
            *reinterpret_cast<f32x4*>(part(par, 2, w)) = St;
        }
        __syncthreads();

        // E[4g + r][c] = sum of the partials - V, the same sum in every wave
        f32x4 E = *reinterpret_cast<const f32x4*>(part(par, 0, 0));
#pragma unroll
        for (int x = 1; x < kWaves; ++x)
            E += *reinterpret_cast<const f32x4*>(part(par, 0, x));
        E -= vv;
        f32x4 Ep;
        if constexpr (kPro)     // rows 4g + r scale by their own step sizes
            Ep = -(*reinterpret_cast<const f32x4*>(sl + L::kOffEta + 4 * g) * E);
        else
            Ep = -et * E;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Wr = mfma(kt[r], Ep[r], Wr);

        if (!kMaps) {
            f32x4 Rs = *reinterpret_cast<const f32x4*>(part(par, 1, 0));
            f32x4 Ss = *reinterpret_cast<const f32x4*>(part(par, 2, 0));
#pragma unroll
            for (int x = 1; x < kWaves; ++x) {
                Rs += *reinterpret_cast<const f32x4*>(part(par, 1, x));
                Ss += *reinterpret_cast<const f32x4*>(part(par, 2, x));
            }
            // lane (c = t, g) holds S[t][s = 4g + r]: keep s <= t (none with
            // the chunk-start read)
            const bool keep = !(kPro && pro.read_start);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Ss[r] = keep && 4 * g + r <= c ? Ss[r] : 0.f;
            f32x4 Yv = Rs;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Yv = mfma(Ss[r], Ep[r], Yv);
            // Y[t0 + 4g + w][16J + c]; rows past the segment fall outside the buffer
            const float yw = w == 0 ? Yv[0] : w == 1 ? Yv[1] : w == 2 ? Yv[2] : Yv[3];
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yw), ry,
                                                  ((ch * kB + 4 * g + w) * kD + 16 * J + c) * 4, 0, 0);
        }
    };

    if (kSplit && nchunks > 0) {
        if (stager) {
            StageRegs ring[kRing];
#pragma unroll
            for (int q = 0; q < kRing; ++q)
                load_stage(ring[q], q);
            write_stage(ring[0], 0);
            write_stage(ring[1], 1);
            load_stage(ring[0], kRing);
            load_stage(ring[1], kRing + 1);
            __syncthreads();
            // barrier ch (the compute waves' barrier of chunk ch), then chunk
            // ch + 2 into its slot (last read by chunk ch - 1) and its register
            // set reloaded with chunk ch + 2 + kRing
            auto advance = [&](int ch, StageRegs& set) {
                __syncthreads();
                write_stage(set, ch + 2);
                load_stage(set, ch + 2 + kRing);
            };
            int c0 = 0;
            for (; c0 + kRing <= nchunks; c0 += kRing) {
#pragma unroll
                for (int p = 0; p < kRing; ++p)
                    advance(c0 + p, ring[(p + 2) % kRing]);
            }
#pragma unroll
            for (int p = 0; p < kRing; ++p) {
                if (c0 + p >= nchunks)   // uniform: the scan is done
                    break;
                advance(c0 + p, ring[(p + 2) % kRing]);
            }
            return;
        }
        __syncthreads();                 // chunks 0 and 1 are in LDS
        asm volatile("" : "+v"(Wr));     // the start state is in registers before the loop
        for (int ch = 0; ch < nchunks; ++ch)
            chunk_step(ch);
    } else if (nchunks > 0) {
        StageRegs ring[kRing];
#pragma unroll
        for (int q = 0; q < kRing; ++q)
            load_stage(ring[q], q);
        write_stage(ring[0], 0);
        write_stage(ring[1], 1);
        load_stage(ring[0], kRing);
        load_stage(ring[1], kRing + 1);
        __syncthreads();
        // chunk ch, then chunk ch + 2 into its slot and its register set
        // reloaded with chunk ch + 2 + kRing (p = ch mod kRing)
        auto advance = [&](int ch, StageRegs& set) {
            chunk_step(ch);
            write_stage(set, ch + 2);
            load_stage(set, ch + 2 + kRing);
        };
        // full rounds without exits, then the last partial round
        int c0 = 0;
        for (; c0 + kRing <= nchunks; c0 += kRing) {
#pragma unroll
            for (int p = 0; p < kRing; ++p)
                advance(c0 + p, ring[(p + 2) % kRing]);
        }
#pragma unroll
        for (int p = 0; p < kRing; ++p) {
            if (c0 + p >= nchunks)       // uniform: the scan is done
                break;
            advance(c0 + p, ring[(p + 2) % kRing]);
        }
    }

    float* wo;
    if (kMaps)
        wo = maps + ((u * (nseg - 1) + s) * 2 + half) * kD * kD;
    else if (s == nseg - 1)
        wo = W_out + u * kD * kD;
    else
        return;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        wo[(16 * w + 4 * g + r) * kD + 16 * J + c] = Wr[r];
}

}  // namespace

bool linear_cols_f32_supports(const LinearArgs& a)
{
    const int64_t max_tokens = (int64_t{1} << 31) / (kD * 4) - kB * (kRing + 4);
    return a.dtype == 0 && a.d == kD && a.b == kB && a.T <= max_tokens;
}

namespace {

template <bool kPro>
hipError_t launch_cols(const LinearArgs& a, const SegmentPlan& p)
{
    const auto* q = static_cast<const float*>(a.Q);
    const auto* k = static_cast<const float*>(a.K);
    const auto* v = static_cast<const float*>(a.V);
    auto* y = static_cast<float*>(a.Y);
    const int H = static_cast<int>(a.H), T = static_cast<int>(a.T);
    const int seg_len = static_cast<int>(p.nseg > 1 ? p.seg_len : (a.T + kB - 1) / kB * kB);
    const int64_t units = a.B * a.H;
    if (p.nseg > 1) {
        const dim3 grid(static_cast<unsigned>(placed_grid(units, 2 * kSlices * (p.nseg - 1))));
        hipLaunchKernelGGL((linear_cols_f32_kernel<true, kPro>), grid, dim3(kThreads), 0, a.stream, q,
                           k, v, a.W0, a.w0_per_batch, a.eta, H, T, units, seg_len, p.nseg, p.maps,
                           p.wstart, y, a.W_out, 0, a.pro);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        if (p.starts_only)               // every start state, for a caller that needs them
            return launch_linear_combine(a, p);
    }
    // segments compose their start states from the maps and the copy of W0
    const dim3 grid(static_cast<unsigned>(placed_grid(units, kSlices * p.nseg)));
    hipLaunchKernelGGL((linear_cols_f32_kernel<false, kPro>), grid, dim3(kPro ? 2 * kThreads : kThreads), 0,
                       a.stream, q, k,
                       v, a.W0, a.w0_per_batch, a.eta, H, T, units, seg_len, p.nseg, p.maps,
                       p.wstart, y, a.W_out, 1, a.pro);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_cols_f32(const LinearArgs& a, const SegmentPlan& p)
{
    return a.pro.active() ? launch_cols<true>(a, p) : launch_cols<false>(a, p);
}

}  // namespace ttt
