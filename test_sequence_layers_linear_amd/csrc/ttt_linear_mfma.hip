// ttt_linear_mfma.hip -- TTT-Linear dual-form scan on MFMA for bf16 Q/K/V,
// head dim d = 64, mini-batch b = 16, fp32 fast weights.
//
// Per chunk of 16 tokens (W = chunk-start weights, row-vector form z W):
//     E' = eta (V - K W)                 (= -eta E, the scaled residual)
//     Y  = Q W + tril(Q K^T) E'          (= Q W - eta tril(Q K^T) E)
//     W  = W + K^T E'                    (= W - eta K^T E)
// the dual form of mini-batch gradient descent ("Test-Time Training Layers:
// How Inner-Loop Gradient Descent Replaces the Transformer KV Cache ...",
// section "Hardware Parallelization: The Dual Form and Mini-Batch GPU
// Acceleration"; the dual-form paragraph of the ren-xubin.github.io essay).
//
// Work split.  One workgroup (4 waves) per (batch, head) chain.  The loss
// 1/2 sum_j (k . W[:, j] - v_j)^2 separates over output columns j, so wave w
// owns the 16 columns [16w, 16w + 16) of W outright and no partial result
// ever moves between waves; the waves share only the staged inputs.  (The
// segment maps and the scan with the input prologue add waves that only
// stage: see the kernel's comment.)
//
// Register dataflow (16x16 MFMA layouts; lane l, c = l % 16, g = l / 16):
//   C/D tile    : lane holds rows 4g..4g+3 of column c.
//   A operand   : lane holds row c, k-slots of group g.
//   B operand   : lane holds column c, k-slots of group g.
// The W slice is kept as the fp32 accumulator of the update MFMA, four 16-row
// tiles mt = 0..3.  Row m of tile mt is input index i = rho(mt, m) with
//     rho(mt, m) = 32 (mt / 2) + 8 (m / 4) + 4 (mt % 2) + m % 4,
// chosen so that the accumulator registers of tiles 2s and 2s+1, rounded to
// bf16, ARE the B operand of a 16x16x32 product over i in [32s, 32s + 32)
// with k-slot (g, e) <-> i = 32s + 8g + e: one contiguous 16-byte segment of
// a K or Q row per lane.  So
//   R    = K W_J - V    : A = K rows, B = W registers; V enters transposed
//                         through a product of its row tile with -I
//   Y^T  = W_J^T Q^T + E'^T S^T : A = the same W registers, B = Q rows
//   S^T  = K Q^T        : lands in exactly the B layout of E'^T S^T
//   E'   = -eta R (C layout) is at once the B operand of the update and the
//        A operand of E'^T S^T
//   W   += K^T E'       : A = K^T, transposed on its way out of LDS
//                         (ds_read_b64_tr_b16 on the row-major K tile)
// Y^T comes out with 4 consecutive columns of one token per lane (one 8-byte
// store).  Only R -> E' -> update -> bf16(W) is a dependent chain per chunk;
// the plain scan runs the second chunk's readout (S^T, Y^T, the store) at
// the start of the next stage, while that stage's LDS reads are in flight.
//
// Memory.  Q, K, V stream from HBM exactly once per chain.  A stage is two
// chunks (32 tokens); for each stage wave w loads rows [8w, 8w + 8) of the
// stage's K, Q and V with fully coalesced 16-byte-per-lane buffer loads (one
// 1 KB row block per instruction) into registers, and later writes them to
// one slot of a 3-slot LDS ring: K, Q, V row-major with the 16-byte segments
// of row r XOR-swizzled by r % 8 (conflict-free operand reads).  Loads run 3
// to 6 stages ahead in two fixed register sets, A and B (while one set is
// consumed the other is in flight), so the compiler can wait on exactly the
// set it needs.  One barrier per stage: at stage s every
// wave writes stage s + 1 into slot (s + 1) % 3, meets the barrier, then
// computes stage s from slot s % 3; the slot being written was last read at
// stage s - 2, before the previous barrier.  Per-chain buffer resources are
// sized to the chain's T tokens, so rows past the end read as zero (an
// all-zero chunk leaves W unchanged) and stores past the end are dropped:
// there are no tail branches.
#include <type_traits>

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
constexpr int kSet = 6;                 // bound on the stages per register set (two sets)
constexpr int kSlots = 3;               // LDS ring slots (kSet * 2 % kSlots == 0)
// LDS layout of one chunk inside a stage slot (bytes)
constexpr int kOffK = 0;
constexpr int kOffQ = kOffK + kB * kRowBytes;        // 2048
constexpr int kOffV = kOffQ + kB * kRowBytes;        // 4096
constexpr int kChunkBytes = kOffV + kB * kRowBytes;  // 6144
constexpr int kSlotBytes = kChunkBytes * kStageChunks;

static_assert((2 * kSet) % kSlots == 0, "slot index must be static inside the loop");

// One wave's share of one stage: rows [8w, 8w + 8) of the stage's K, Q, V;
// lane l holds row 8w + l / 8, 16-byte segment l % 8.
struct StageRegs {
    u32x4 k, q, v;
    uint32_t eta;      // step size of this lane's token (prologue only)
};


// kMaps = false: the scan of segment s of a chain (Y rows of the segment; the
//   last segment also writes W_out), started from W0 (one segment) or from
//   the segment's start state in wstart.
// kMaps = true: the affine map W_end = M W_start + N of segment s < nseg - 1,
//   12 waves: waves 0-3 (half 0) run the scan from W = I with V = 0 (giving
//   M), waves 4-7 (half 1) from W = 0 with the segment's V (giving N); both
//   halves share the staged K, which waves 8-11 load and write to LDS (as
//   the K group of the prologue scan below; with the prologue they also
//   LayerNorm it and stage the step sizes).  No Q, no Y.
// With nseg > 1 the blocks of chain u all run on XCD u % 8 (see xcd_block),
// so the maps, start states and scans of a chain meet in one L2.
// kPro: the input prologue (Prologue in ttt_internal.h) is applied while the
//   inputs are staged: K and Q rows LayerNorm'd over the head dim in fp32 and
//   rounded to bf16, and each token's step size written after the stage in
//   LDS, where it scales its row of the residual: E'[t] = -eta_t R[t] (the
//   head's eta when no per-token step sizes are given); with read_start every
//   token reads out with the chunk-start W (the tril term is dropped).
// kMaps = false with kPro: 12 waves in two roles.  Waves 0-3 compute (as in
//   the plain scan); waves 4-11 only stage, one stage ahead of the compute
//   waves: waves 4-7 load K, V and the step sizes and LayerNorm K, waves
//   8-11 load and LayerNorm Q, and both write their rows to LDS.  So the
//   normalisation's VALU work runs beside the chunk chain on the same SIMDs
//   (one wave of each kind per SIMD) instead of inside it.  The roles run
//   loops of their own with one barrier per stage each.
// kStream: the inputs are loaded non-temporally (used when a call's Q, K, V
//   exceed the last-level cache, so that caching them only evicts other
//   lines: 278 us against 288 us per call on B2 H24 T32768 with a cold
//   cache, where 75 MB of inputs that the cache can hold load 10% slower
//   when they are re-read warm).
// One workgroup's work: segment s of chain u (segment 0 holds first_len
// tokens, the others seg_len each).  end_to_wstart: the scan of segment 0
// writes its end state as the start state of segment 1 (the first launch of
// the fused layout, see linear_fused_kernel).
template <bool kMaps, bool kPro, bool kStream>
__device__ __forceinline__ void
linear_body(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
            const uint16_t* __restrict__ V, const float* W0, int w0_per_batch,
            const float* __restrict__ eta, int H, int T, int seg_len, int first_len, int nseg,
            float* maps, float* wstart, uint16_t* __restrict__ Y, float* W_out,
            const Prologue& pro, int64_t u, int s, bool end_to_wstart)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int lane = threadIdx.x & 63;
    const int w = (threadIdx.x >> 6) & (kWaves - 1);
    // wave-uniform role flags, made scalar so that the compiler branches on
    // them instead of masking lanes
    constexpr bool kSplit = kPro || kMaps;
    // (half is 2 on the staging waves 8-11 of a maps block)
    const int half = kMaps ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 8)) : 0;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const bool stager = kSplit ? wave >= (kMaps ? 2 : 1) * kWaves : (!kMaps || wave < kWaves);
    const int c = lane & 15;
    const int g = lane >> 4;
    const int col = 16 * w + c;          // this lane's column of W

    const int h = static_cast<int>(u % H);
    const float et = eta[h];
    const int t_begin = s == 0 ? 0 : first_len + (s - 1) * seg_len;
    const int t_len = max(0, min(s == 0 ? first_len : seg_len, T - t_begin));
    // map j of chain u: M at maps + (u (nseg - 1) + j) 2 64 64, N right after
    auto map_ptr = [&](int j) { return maps + ((u * (nseg - 1) + j) * 2) * kD * kD; };

    // fast weights: Wacc[mt][r] = W[rho(mt, 4g + r)][col]
    f32x4 Wacc[4];
    if (kMaps) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Wacc[mt][r] = (half == 0 && rho(mt, 4 * g + r) == col) ? 1.0f : 0.0f;
    } else if (!kSplit || !stager) {
        // W0 itself only for the only segment and for segment 0 in the fused
        // layout's first launch, which runs before any segment writes W_out
        // (W_out may be W0); otherwise the start states of the composition
        // (its copy of W0 for segment 0)
        const bool from_w0 = nseg == 1 || end_to_wstart;
        const float* w0 = from_w0 ? W0 + (w0_per_batch ? u : h) * kD * kD
                                  : wstart + (u * nseg + s) * kD * kD;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Wacc[mt][r] = w0[rho(mt, 4 * g + r) * kD + col];
    }

    // -I as the B operand of a 16x16x16 product: B[k = 4g + r][n = c] = -(k == n)
    bf16x4 neg_eye;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        neg_eye[r] = static_cast<__bf16>(4 * g + r == c ? -1.0f : 0.0f);

    const int64_t base = (u * static_cast<int64_t>(T) + t_begin) * kD;
    const int64_t seg_bytes = static_cast<int64_t>(t_len) * kD * 2;
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(Q + base, kMaps ? 0 : seg_bytes);
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(K + base, seg_bytes);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(V + base, seg_bytes);
    const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(Y + base, kMaps ? 0 : seg_bytes);

    const int nstages = (t_len + kStageTokens - 1) / kStageTokens;
    // a slot also holds the stage's 32 step sizes when the prologue is on
    constexpr int kSlotB = kPro ? kSlotBytes + kStageTokens * 4 : kSlotBytes;
    // stages per register set: every instantiation prefetches 3-6 stages
    // ahead (the bound on T allows for 6-12).  6-12 ahead was slower: the
    // plain scan 48.1 against 42.6 us on B8 H12 T2048 with a cold cache and
    // 269 against 258 us on B2 H24 T32768; with the prologue 63.7 against
    // 57.9 and 341 against 321 us.
    constexpr int kSetK = kSet / 2;
    static_assert((2 * kSetK) % kSlots == 0, "slot index must be static inside the loop");
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // staging: this lane's row inside the stage and its 16-byte segment
    const int st_row = 8 * w + (lane >> 3);             // 0..31
    const int st_seg = lane & 7;
    // prologue: LayerNorm gamma, beta of this lane's 8 columns 8 st_seg .. +7
    const bool use_tok = kPro && pro.eta_tok != nullptr;
    const bool ln_k = kPro && pro.ln_k != nullptr;
    const bool ln_q = kPro && !kMaps && pro.ln_q != nullptr;
    float gk[8], bk[8], gq[8], bq[8];
    if constexpr (kPro) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            gk[e] = ln_k ? pro.ln_k[(2 * h) * kD + 8 * st_seg + e] : 1.f;
            bk[e] = ln_k ? pro.ln_k[(2 * h + 1) * kD + 8 * st_seg + e] : 0.f;
            gq[e] = ln_q ? pro.ln_q[(2 * h) * kD + 8 * st_seg + e] : 1.f;
            bq[e] = ln_q ? pro.ln_q[(2 * h + 1) * kD + 8 * st_seg + e] : 0.f;
        }
    }
    const __amdgpu_buffer_rsrc_t reta =
        buffer_rsrc(use_tok ? pro.eta_tok + u * static_cast<int64_t>(T) + t_begin : eta,
                   use_tok ? static_cast<int64_t>(t_len) * 4 : 0);
    auto load_stage = [&](StageRegs& o, int stage) {
        if (!stager)
            return;
        const int off = (stage * kStageTokens + st_row) * kRowBytes + st_seg * 16;
        constexpr int kPolicy = kStream ? kNonTemporal : 0;
        o.k = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kPolicy);
        if (!kMaps)
            o.q = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, kPolicy);
        o.v = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kPolicy);
        if (kPro)             // a zero-sized resource without per-token step sizes
            o.eta = __builtin_amdgcn_raw_buffer_load_b32(reta, (stage * kStageTokens + st_row) * 4, 0, 0);
    };
    // LayerNorm of a staged row segment (8 bf16 per lane, 8 lanes per row),
    // rounded back to bf16
    auto norm = [&](u32x4 x, const float (&gm)[8], const float (&bt)[8], bool valid) {
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[2 * e] = __uint_as_float(x[e] << 16);
            f[2 * e + 1] = __uint_as_float(x[e] & 0xffff0000u);
        }
        layernorm_row<8, 8>(f, gm, bt, pro.ln_eps, valid);
        const bf16x8 r = pack8(f32x4{f[0], f[1], f[2], f[3]}, f32x4{f[4], f[5], f[6], f[7]});
        return __builtin_bit_cast(u32x4, r);
    };
    // LayerNorm a stage's rows in their registers, at the end of the stage
    // before the one that writes them to LDS: after that stage's products, so
    // that the scheduler can overlap the two
    auto prep = [&](StageRegs& o, int stage) {
        if constexpr (kPro) {
            if (!stager)
                return;
            const bool valid = stage * kStageTokens + st_row < t_len;
            if (ln_k)
                o.k = norm(o.k, gk, bk, valid);
            if (ln_q)
                o.q = norm(o.q, gq, bq, valid);
        }
    };
    auto write_stage = [&](const StageRegs& o, int slot) {
        if (!stager)
            return;
        if constexpr (kPro) {
            // (the 8 lanes of a row store the same value: no lane branch)
            *reinterpret_cast<float*>(lds + slot * kSlotB + kSlotBytes + 4 * st_row) =
                use_tok ? __uint_as_float(o.eta) : et;
        }
        unsigned char* chunk = lds + slot * kSlotB + (st_row >> 4) * kChunkBytes;
        const int r = st_row & 15;
        *reinterpret_cast<u32x4*>(chunk + kOffK + swz(r, st_seg)) = o.k;
        if (!kMaps)
            *reinterpret_cast<u32x4*>(chunk + kOffQ + swz(r, st_seg)) = o.q;
        *reinterpret_cast<u32x4*>(chunk + kOffV + swz(r, st_seg)) = o.v;
    };

    // Operands of one chunk, read from its LDS tile.
    struct ChunkOps {
        bf16x8 ka0, ka1, qa0, qa1;
        bf16x4 vrow;
        bf16x4 kt[4];
        f32x4 eta4;        // step sizes of tokens 4g .. 4g+3 (prologue)
    };
    auto read_ops = [&](ChunkOps& o, const unsigned char* tile) {
        o.ka0 = *reinterpret_cast<const bf16x8*>(tile + kOffK + swz(c, g));
        o.ka1 = *reinterpret_cast<const bf16x8*>(tile + kOffK + swz(c, 4 + g));
        if (!kMaps) {
            o.qa0 = *reinterpret_cast<const bf16x8*>(tile + kOffQ + swz(c, g));
            o.qa1 = *reinterpret_cast<const bf16x8*>(tile + kOffQ + swz(c, 4 + g));
        }
        o.vrow = *reinterpret_cast<const bf16x4*>(tile + kOffV + swz(c, 2 * w + (g >> 1)) + 8 * (g & 1));
        // K^T operand of the update, transposed on the way out of LDS: lane
        // (c, g) addresses row 4g + c / 4, inputs rho(mt, 4 (c % 4) .. + 3) (8
        // contiguous bytes) and receives K[4g + r][rho(mt, c)], r = 0..3
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            o.kt[mt] = read_tr16(tile + kOffK + swz(4 * g + (c >> 2), 4 * (mt >> 1) + (c & 3)) + 8 * (mt & 1));
    };

    // Readout of one chunk, rows t0 .. t0 + 15 of Y, from its K and Q
    // operands, the bf16 chunk-start W slice (b0, b1) and E' (eb): off the
    // chain, so the plain scan runs the second chunk of a stage at the start
    // of the next stage, where it fills the wait for that stage's LDS reads
    // (41.4 against 42.6 us on B8 H12 T2048, 247 against 258 us on B2 H24
    // T32768, both with a cold cache; the same results bit for bit).
    auto readout = [&](const bf16x8& ka0, const bf16x8& ka1, const bf16x8& qa0,
                       const bf16x8& qa1, const bf16x8& b0, const bf16x8& b1, const bf16x4& eb,
                       int t0) {
        // S^T = K Q^T, Y^T partial = W_J^T Q^T
        f32x4 St = mfma32(ka0, qa0, zero);
        St = mfma32(ka1, qa1, St);
        f32x4 Yt = mfma32(b0, qa0, zero);
        Yt = mfma32(b1, qa1, Yt);

        // S^T masked: lane (c = t, g) holds S[t][t' = 4g + r]; keep t' <= t
        f32x4 Sm;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Sm[r] = (4 * g + r <= c) ? St[r] : 0.f;
        // (the chunk-start read drops the intra-chunk term: zero operand)
        const bf16x4 sb = (kPro && pro.read_start) ? bf16x4{} : pack4(Sm);
        Yt = mfma16_as32(eb, sb, Yt);

        // Y[t0 + c][16w + 4g .. +3]; rows past the segment fall outside the buffer.
        const bf16x4 yb = pack4(Yt);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, yb), ry,
                                              ((t0 + c) * kD + 16 * w + 4 * g) * 2, 0, 0);
    };
    // a readout held over to the next stage
    struct Pending {
        bf16x8 ka0, ka1, qa0, qa1, b0, b1;
        bf16x4 eb;
    };
    Pending pend;
    int pend_t0 = 0;

    // One chunk of the scan, tokens t0 onwards; kDefer (plain scan only):
    // keep its readout's operands in `pend` instead of reading out.
    auto step = [&](const ChunkOps& o, int t0, auto defer) {
        constexpr bool kDefer = decltype(defer)::value && !kSplit;
        // bf16 copy of the W slice at the chunk start: the B operand of K W_J
        // and the A operand of W_J^T Q^T (k-slot (g, e) of pair s <-> input
        // index 32s + 8g + e)
        const bf16x8 b0 = pack8(Wacc[0], Wacc[1]);
        const bf16x8 b1 = pack8(Wacc[2], Wacc[3]);

        // R = K W_J - V (C layout: rows t = 4g + r, column col); the -I
        // product is issued in the 16x16x32 shape of the chain it starts
        // (the M half, half 0, of a maps block has V = 0: its V operand is
        // zeroed rather than the product skipped, since an MFMA inside an
        // EXEC-masked region still executes)
        const bf16x4 vrow = (kMaps && half == 0) ? bf16x4{} : o.vrow;
        f32x4 R = mfma16_as32(vrow, neg_eye, zero);
        R = mfma32(o.ka0, b0, R);
        R = mfma32(o.ka1, b1, R);

        // E' = eta (V - K W) = -eta R (row t scaled by its own step size
        // with the prologue)
        const bf16x4 eb = pack4(kPro ? -(o.eta4 * R) : -et * R);

        // W += K^T E'
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            Wacc[mt] = mfma16(o.kt[mt], eb, Wacc[mt]);

        if constexpr (kDefer) {
            pend = Pending{o.ka0, o.ka1, o.qa0, o.qa1, b0, b1, eb};
            pend_t0 = t0;
        } else if constexpr (!kMaps) {
            readout(o.ka0, o.ka1, o.qa0, o.qa1, b0, b1, eb, t0);
        }
    };
    auto flush = [&]() {
        readout(pend.ka0, pend.ka1, pend.qa0, pend.qa1, pend.b0, pend.b1, pend.eb, pend_t0);
    };

    // Stage s: publish stage s + 1 (held in `next`), then compute stage s.
    auto process = [&](const StageRegs& next, int s, int slot, StageRegs& ahead) {
        write_stage(next, (slot + 1) % kSlots);
        __syncthreads();
        const unsigned char* sl = lds + slot * kSlotB;
        ChunkOps o0, o1;
        read_ops(o0, sl);
        read_ops(o1, sl + kChunkBytes);
        if constexpr (kPro) {
            o0.eta4 = *reinterpret_cast<const f32x4*>(sl + kSlotBytes + 16 * g);
            o1.eta4 = *reinterpret_cast<const f32x4*>(sl + kSlotBytes + 64 + 16 * g);
        }
        if constexpr (!kSplit)
            if (s > 0)                   // the previous stage's second readout
                flush();
        step(o0, s * kStageTokens, std::false_type{});
        step(o1, s * kStageTokens + kB, std::true_type{});
        prep(ahead, s + 2);
    };

    if (kSplit && nstages > 0) {
        if (stager) {
            // waves 4-7 (kgrp) and 8-11 run the same instruction stream on
            // different buffers: x is K or Q, y is V or nothing, e the step
            // sizes or nothing (a zero-sized resource reads as zero)
            const bool kgrp = kMaps || wave < 2 * kWaves;
            const __amdgpu_buffer_rsrc_t rx = buffer_rsrc((kgrp ? K : Q) + base, seg_bytes);
            const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(V + base, kgrp ? seg_bytes : 0);
            const __amdgpu_buffer_rsrc_t re =
                buffer_rsrc(use_tok ? pro.eta_tok + u * static_cast<int64_t>(T) + t_begin : eta,
                           use_tok && kgrp ? static_cast<int64_t>(t_len) * 4 : 0);
            const bool ln_x = kgrp ? ln_k : ln_q;
            const int off_x = kgrp ? kOffK : kOffQ;
            float gx[8], bx[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                gx[e] = kgrp ? gk[e] : gq[e];
                bx[e] = kgrp ? bk[e] : bq[e];
            }
            struct Rows {
                u32x4 x, y;
                uint32_t e;
            };
            auto load = [&](Rows& o, int stage) {
                const int off = (stage * kStageTokens + st_row) * kRowBytes + st_seg * 16;
                o.x = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
                o.y = __builtin_amdgcn_raw_buffer_load_b128(ry, off, 0, 0);
                if constexpr (kPro)
                    o.e = __builtin_amdgcn_raw_buffer_load_b32(re, (stage * kStageTokens + st_row) * 4, 0, 0);
            };
            // LayerNorm'd rows of stage `stage` into LDS slot `slot`
            auto put = [&](Rows& o, int stage, int slot) {
                if (ln_x)
                    o.x = norm(o.x, gx, bx, stage * kStageTokens + st_row < t_len);
                unsigned char* chunk = lds + slot * kSlotB + (st_row >> 4) * kChunkBytes;
                const int r = st_row & 15;
                *reinterpret_cast<u32x4*>(chunk + off_x + swz(r, st_seg)) = o.x;
                if (kgrp) {
                    *reinterpret_cast<u32x4*>(chunk + kOffV + swz(r, st_seg)) = o.y;
                    // (the 8 lanes of a row store the same value)
                    if constexpr (kPro)
                        *reinterpret_cast<float*>(lds + slot * kSlotB + kSlotBytes + 4 * st_row) =
                            use_tok ? __uint_as_float(o.e) : et;
                }
            };
            // stage s + 1 goes to LDS before barrier s; loads run 3 to 6
            // stages ahead in two register sets, as in the plain scan
            Rows setA[kSetK], setB[kSetK];
            {
                Rows first;
                load(first, 0);
                put(first, 0, 0);
            }
#pragma unroll
            for (int p = 0; p < kSetK; ++p)
                load(setA[p], 1 + p);
            for (int s0 = 0; s0 < nstages; s0 += 2 * kSetK) {
#pragma unroll
                for (int p = 0; p < kSetK; ++p)
                    load(setB[p], s0 + kSetK + 1 + p);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int p = 0; p < kSetK; ++p) {
                    if (s0 + p >= nstages)       // uniform: the scan is done
                        goto done;
                    put(setA[p], s0 + p + 1, (p + 1) % kSlots);
                    __syncthreads();
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int p = 0; p < kSetK; ++p)
                    load(setA[p], s0 + 2 * kSetK + 1 + p);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int p = 0; p < kSetK; ++p) {
                    if (s0 + kSetK + p >= nstages)
                        goto done;
                    put(setB[p], s0 + kSetK + p + 1, (kSetK + p + 1) % kSlots);
                    __syncthreads();
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // the start state is in registers before the loop (otherwise the
            // wait for it lands inside the loop and waits for the Y stores)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                asm volatile("" : "+v"(Wacc[mt]));
            for (int s0 = 0; s0 < nstages; s0 += kSlots) {
#pragma unroll
                for (int p = 0; p < kSlots; ++p) {
                    if (s0 + p >= nstages)
                        goto done;
                    __syncthreads();
                    const unsigned char* sl = lds + p * kSlotB;
                    ChunkOps o0, o1;
                    read_ops(o0, sl);
                    read_ops(o1, sl + kChunkBytes);
                    if constexpr (kPro) {
                        o0.eta4 = *reinterpret_cast<const f32x4*>(sl + kSlotBytes + 16 * g);
                        o1.eta4 = *reinterpret_cast<const f32x4*>(sl + kSlotBytes + 64 + 16 * g);
                    }
                    step(o0, (s0 + p) * kStageTokens, std::false_type{});
                    step(o1, (s0 + p) * kStageTokens + kB, std::false_type{});
                }
            }
        }
    } else if (nstages > 0) {
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
        // stages s0 .. s0 + 2 kSetK - 1 per iteration; setA holds s0 + 1 .. s0 + kSetK
        for (int s0 = 0; s0 < nstages; s0 += 2 * kSetK) {
#pragma unroll
            for (int p = 0; p < kSetK; ++p)
                load_stage(setB[p], s0 + kSetK + 1 + p);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = 0; p < kSetK; ++p) {
                if (s0 + p >= nstages)       // uniform: the scan is done
                    goto done;
                process(setA[p], s0 + p, p % kSlots, p + 1 < kSetK ? setA[p + 1] : setB[0]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = 0; p < kSetK; ++p)
                load_stage(setA[p], s0 + 2 * kSetK + 1 + p);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = 0; p < kSetK; ++p) {
                if (s0 + kSetK + p >= nstages)
                    goto done;
                process(setB[p], s0 + kSetK + p, (kSetK + p) % kSlots,
                        p + 1 < kSetK ? setB[p + 1] : setA[0]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
done:
    if constexpr (!kSplit)
        if (nstages > 0)
            flush();
    if (kSplit && stager)
        return;

    float* wo;
    if (kMaps)
        wo = map_ptr(s) + half * kD * kD;
    else if (s == nseg - 1)
        wo = W_out + u * kD * kD;
    else if (end_to_wstart)
        wo = wstart + (u * nseg + 1) * kD * kD;
    else
        return;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            wo[rho(mt, 4 * g + r) * kD + col] = Wacc[mt][r];
}

// The scans or maps of the plan: segments seg_base .. of every chain (maps:
// segments 0 .. nseg - 2), nb workgroups per chain placed by xcd_block.
template <bool kMaps, bool kPro, bool kStream>
__global__ void __launch_bounds__(kPro || kMaps ? 3 * kThreads : kThreads, 1)
linear_mfma_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, const float* W0, int w0_per_batch,
                   const float* __restrict__ eta, int H, int T, int64_t units, int seg_len,
                   int first_len, int nseg, int seg_base, float* maps, float* wstart,
                   uint16_t* __restrict__ Y, float* W_out, Prologue pro)
{
    int64_t u = blockIdx.x;
    int s = 0;
    if (nseg > 1) {
        xcd_block(blockIdx.x, kMaps ? nseg - 1 : nseg - seg_base, units, u, s);
        if (u >= units)                  // padding of the XCD placement
            return;
    }
    linear_body<kMaps, kPro, kStream>(Q, K, V, W0, w0_per_batch, eta, H, T, seg_len, first_len,
                                      nseg, maps, wstart, Y, W_out, pro, u, s + seg_base, false);
}

// First launch of the fused layout: per chain, workgroup 0 scans segment 0
// (Y rows and its end state, the start state of segment 1) while workgroups
// 1 .. nseg - 2 form the maps of segments 1 .. nseg - 2, so segment 0 needs no
// map.  Both roles run 12 waves: the scan in the staged form of the prologue
// scan (with the prologue off unless kPro: the same products as the plain
// scan, bit for bit), the maps as in the unfused layout (kPro: with the
// LayerNorm of K and the step sizes).
template <bool kPro, bool kStream>
__global__ void __launch_bounds__(3 * kThreads, 1)
linear_fused_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                    const uint16_t* __restrict__ V, const float* W0, int w0_per_batch,
                    const float* __restrict__ eta, int H, int T, int64_t units, int seg_len,
                    int first_len, int nseg, float* maps, float* wstart,
                    uint16_t* __restrict__ Y, float* W_out, Prologue pro)
{
    int64_t u = blockIdx.x;
    int s = 0;
    xcd_block(blockIdx.x, nseg - 1, units, u, s);
    if (u >= units)
        return;
    if (s == 0)
        linear_body<false, true, kStream>(Q, K, V, W0, w0_per_batch, eta, H, T, seg_len,
                                          first_len, nseg, maps, wstart, Y, W_out,
                                          kPro ? pro : Prologue{}, u, 0, true);
    else
        linear_body<true, kPro, kStream>(Q, K, V, W0, w0_per_batch, eta, H, T, seg_len,
                                         first_len, nseg, maps, wstart, Y, W_out,
                                         kPro ? pro : Prologue{}, u, s, false);
}

}  // namespace

bool linear_mfma_supports(const LinearArgs& a)
{
    // per-chain byte offsets, including the loads past the end, are 32-bit
    const int64_t max_tokens = (int64_t{1} << 31) / (kD * 2) - kStageTokens * (3 * kSet + 2);
    return a.dtype == 1 && a.d == kD && a.b == kB && a.T <= max_tokens;
}

namespace {

template <bool kPro, bool kStream>
hipError_t launch_bf16(const LinearArgs& a, const SegmentPlan& p)
{
    const auto* q = static_cast<const uint16_t*>(a.Q);
    const auto* k = static_cast<const uint16_t*>(a.K);
    const auto* v = static_cast<const uint16_t*>(a.V);
    auto* y = static_cast<uint16_t*>(a.Y);
    const int H = static_cast<int>(a.H), T = static_cast<int>(a.T);
    const int seg_len = static_cast<int>(p.seg_len);
    const int first_len = static_cast<int>(p.first());
    const int64_t units = a.B * a.H;
    const int lds = kSlots * (kPro ? kSlotBytes + kStageTokens * 4 : kSlotBytes);
    int seg_base = 0;
    if (p.nseg > 1) {
        const dim3 grid(static_cast<unsigned>(placed_grid(units, p.nseg - 1)));
        if (p.fused) {
            // (the staged scan's slots also hold the step sizes)
            hipLaunchKernelGGL((linear_fused_kernel<kPro, kStream>), grid, dim3(3 * kThreads),
                               kSlots * (kSlotBytes + kStageTokens * 4), a.stream, q, k, v, a.W0,
                               a.w0_per_batch, a.eta, H, T, units, seg_len, first_len, p.nseg,
                               p.maps, p.wstart, y, a.W_out, a.pro);
            seg_base = 1;
        } else {
            hipLaunchKernelGGL((linear_mfma_kernel<true, kPro, kStream>), grid, dim3(3 * kThreads),
                               lds, a.stream, q, k, v, a.W0, a.w0_per_batch, a.eta, H, T, units,
                               seg_len, first_len, p.nseg, 0, p.maps, p.wstart, y, a.W_out, a.pro);
        }
        hipError_t e = hipGetLastError();
        if (e == hipSuccess)
            e = launch_linear_combine(a, p);
        if (e != hipSuccess || p.starts_only)
            return e;
    }
    const dim3 grid(static_cast<unsigned>(p.nseg > 1 ? placed_grid(units, p.nseg - seg_base) : units));
    hipLaunchKernelGGL((linear_mfma_kernel<false, kPro, kStream>), grid, dim3(kPro ? 3 * kThreads : kThreads), lds,
                       a.stream, q, k, v,
                       a.W0, a.w0_per_batch, a.eta, H, T, units, seg_len, first_len, p.nseg, seg_base,
                       p.maps, p.wstart, y, a.W_out, a.pro);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_mfma(const LinearArgs& a, const SegmentPlan& p)
{
    const bool stream = a.B * a.H * a.T * a.d * 2 * 3 > kLastLevelCacheBytes;
    if (a.pro.active())
        return stream ? launch_bf16<true, true>(a, p) : launch_bf16<true, false>(a, p);
    return stream ? launch_bf16<false, true>(a, p) : launch_bf16<false, false>(a, p);
}

}  // namespace ttt
