// ttt_linear_backward_bf16.hip -- backward of the TTT-Linear dual-form scan
// for bf16 Q/K/V on bf16 MFMA (d = 64, b = 16; fp32 state, cotangent and
// accumulation).  Same recurrence, segments and work split as the fp32
// kernel in ttt_linear_backward.hip (see there for the derivation):
//     P  = A^T dY + K G'      dE = -eta P      deta += -<P, E>
//     dA = -eta tril(dY E^T)  dQ = dY W^T + dA K
//     dK = -eta (P W^T + E G'^T) + dA^T Q      dV = eta P
//     G  = G' + Q^T dY + K^T dE
// with every product on v_mfma_f32_16x16x32_bf16 (contractions over the
// 64-wide head dim) or v_mfma_f32_16x16x16_bf16 (over the 16 tokens of a
// chunk); operands are rounded to bf16 as in the forward kernel, results
// accumulate in fp32.
//
// Layouts (lane l, c = l % 16, g = l / 16): 16x16x32 A operand lane holds
// A[c][8g .. 8g+7], B operand B[8g .. 8g+7][c]; 16x16x16 A operand A[c][4g ..
// 4g+3], B operand B[4g .. 4g+3][c]; accumulators rows 4g .. 4g+3 of column
// c.  The state W (sweep 1) and the cotangent G keep their 64 x 16 column
// block as four fp32 accumulator tiles mt whose row m is input index
// rho(mt, m) = 32 (mt / 2) + 8 (m / 4) + 4 (mt % 2) + m % 4, so tiles 2s and
// 2s + 1 packed to bf16 are the B operand of a product over the input index
// i in [32 s, 32 s + 32) (k-slot (g, e) <-> i = 32 s + 8 g + e), and the
// 16x16x16 products that update them take A = K^T or Q^T read in the same
// rho order.  An accumulator read as a 16x16x16 A operand is the transpose of
// itself, which gives A^T from S = Q K^T and dA^T from dA.  Products of the
// two shapes never share an accumulator (they are summed in fp32 instead).
//
// LDS (bf16, 16-byte segments of each 128-byte row XOR-swizzled by row):
// a two-slot ring of the chunk's Q, K, dY tiles, W_c^T (one buffer), E and P
// tiles and G'^T for phase B.  Column reads use ds_read_b64_tr_b16: within a
// 16-lane group, lane i receives element i % 4 of the 8-byte block addressed
// by lane 4k + i / 4 as its element k, so lanes addressing rows r0 + j / 4 at
// columns x0 + 4 (j % 4) hand lane i the 4 values X[r0 .. r0 + 3][x0 + i].
// Chunk-start states without storing them: sweep 1 writes each chunk's
// update operand E'_c = bf16(-eta E_c) to the workspace (8 bytes per lane, 2
// KB per chunk) and ends with W of the segment's last chunk in registers;
// sweep 2 walks back from there, W_c = W_{c+1} - K_c^T E'_c, the same
// product with E'_c negated (exact in bf16), so each W_c is the one sweep 1
// passed through up to the fp32 rounding of one add per chunk (no inverse is
// taken and no error is amplified), and its bf16 W_c^T goes to LDS from the
// registers.  A quarter of the 8 KB per chunk that W_c^T in bf16 would take
// each way.
//
// kPro: the input prologue.  Raw Q, K rows are LayerNorm'd (per-head gamma,
// beta over the 64-wide head dim) as they are staged into LDS, keeping the
// normalised rows xh and 1/std per row in the staging threads' registers; a
// step size per token eta_t replaces the head's (E and P scale by row, dA by
// column: dA[t][s] = -eta_s dY_t . E_s); the chunk-start read drops A.  dQ and
// dK of the normalised rows go through LDS to the staging threads, which apply
// the LayerNorm backward to their row segment, store the raw-row gradients
// and sum the gamma, beta gradients; per-token deta_t = -<P_t, E_t> is summed
// over the columns of each wave and then over the waves.
#include "ttt_mfma_ops.h"

namespace ttt {
namespace {

using namespace mfma;

constexpr int kD = 64;
constexpr int kB = 16;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRow = kRowBytes;                 // bytes per bf16 row
constexpr int kTileB = kB * kRow;               // 2048: a 16 x 64 tile
constexpr int kMatB = kD * kRow;                // 8192: a 64 x 64 matrix
constexpr int kSlotQ = 0;
constexpr int kSlotK = kTileB;
constexpr int kSlotDY = 2 * kTileB;
constexpr int kSlotBytes = 3 * kTileB;
constexpr int kFP = 68;                         // padded fp32 row of the dQ, dK tiles

// LDS layout (bytes); kPro adds the slots' step sizes, the fp32 dQ, dK tiles
// of the normalised rows and the per-wave deta_t partial sums.
template <bool kPro>
struct Lay {
    static constexpr int kEta = 2 * kSlotBytes;            // [2 slots][16] eta_t (kPro)
    static constexpr int kW = kEta + (kPro ? 2 * kB * 4 : 0);   // W_c^T [64 j][64 i]
    static constexpr int kE = kW + kMatB;                  // E  [16][64]
    static constexpr int kP = kE + kTileB;                 // P  [16][64]
    static constexpr int kG = kP + kTileB;                 // G'^T [64 j][64 i]
    static constexpr int kRed = kG + kMatB;                // [4] deta partials
    static constexpr int kDQ = kRed + 16;                  // [16][kFP] fp32 (kPro)
    static constexpr int kDK = kDQ + kB * kFP * 4;
    static constexpr int kDeta = kDK + kB * kFP * 4;       // [4 waves][16] (kPro)
    static constexpr int kBytes = kPro ? kDeta + kWaves * kB * 4 : kRed + 16;
    static constexpr int kGMapBytes = kW;                  // the cotangent maps use the slots only
};
static_assert(Lay<false>::kBytes == 32784, "plain layout");
static_assert(2 * Lay<true>::kBytes <= kMaxLdsBytes, "two workgroups per CU");
static_assert(kWaves * 4 * kD * 4 <= 2 * kB * kFP * 4, "the gamma/beta reduction fits the dQ, dK tiles");

__device__ __forceinline__ bf16x8 join(bf16x4 lo, bf16x4 hi)
{
    const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

// (a chain's rows are read through buffer resources: loads past the end read
// zero and stores past it are dropped, so the tokens past T need no branch;
// a memory operation under a branch costs the compiler's wait counts their
// precision, and the stage loads of the chunks ahead must stay in flight)

// byte offset of element x of row r
__device__ __forceinline__ int swz_elem(int r, int x) { return swz(r, x >> 3) + 2 * (x & 7); }

// X[r0 .. r0 + 3][x0 + c] for lane (c, .) of a row-major swizzled tile
// (x0 a multiple of 16)
__device__ __forceinline__ bf16x4 col4(const unsigned char* tile, int r0, int x0, int c)
{
    return read_tr16(tile + swz_elem(r0 + (c >> 2), x0 + 4 * (c & 3)));
}
// X[r0 .. r0 + 3][rho(mt, c)]: the rho-ordered column block of input tile mt
__device__ __forceinline__ bf16x4 col4_rho(const unsigned char* tile, int r0, int mt, int c)
{
    return read_tr16(tile + swz(r0 + (c >> 2), 4 * (mt >> 1) + (c & 3)) + 8 * (mt & 1));
}
__device__ __forceinline__ bf16x8 row8(const unsigned char* tile, int r, int seg)
{
    return *reinterpret_cast<const bf16x8*>(tile + swz(r, seg));
}

struct Stage {
    u32x2 q, k, dy;    // 4 bf16 of row tid / 16, columns 4 (tid % 16) .. +3
    uint32_t v[4];     // V[4g + r][16w + c] of this lane's column: the 4-byte word holding
                       // the bf16 value (a whole word: no extension after the load, so
                       // the value can stay in flight; vneg picks the half)
    u32x2 e;           // E'_c of this lane: sweep 1's update operand of the chunk
    float eta;         // kPro: the step size of row tid / 16 (0 past T)
    bool ok;           // row tid / 16 is a token (< T)
};

__device__ __forceinline__ void unpack4(u32x2 x, float (&f)[4])
{
    f[0] = __uint_as_float(x[0] << 16);
    f[1] = __uint_as_float(x[0] & 0xffff0000u);
    f[2] = __uint_as_float(x[1] << 16);
    f[3] = __uint_as_float(x[1] & 0xffff0000u);
}

template <bool kGMap, bool kPro>
__global__ void __launch_bounds__(kThreads, 2)
linear_backward_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                            const uint16_t* __restrict__ V, const float* __restrict__ W0,
                            int w0_per_batch, const float* __restrict__ eta, int H, int T,
                            int64_t units, int seg_len, int nseg, const float* __restrict__ wstart,
                            const float* __restrict__ gend, const uint16_t* __restrict__ dY,
                            const float* __restrict__ dW_out, uint16_t* __restrict__ dQ,
                            uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                            float* __restrict__ dW0_chain, float* __restrict__ deta_chain,
                            uint16_t* __restrict__ states, float* __restrict__ gmaps,
                            Prologue pro, float* __restrict__ deta_tok, float* __restrict__ dln_chain,
                            const float* __restrict__ fmaps)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    using L = Lay<kPro>;
    constexpr int kOffW = L::kW, kOffE = L::kE, kOffP = L::kP, kOffG = L::kG, kOffRed = L::kRed;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int col = 16 * w + c;

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
    if (kGMap && half == 0 && s < nseg - 1) {
        // The linear part of a segment's cotangent map, the product of the
        // chunks' I - K^T diag(eta) K from the segment's end to its start,
        // is the transpose of the forward map's product of the same
        // symmetric factors in the forward order, which the forward maps
        // launch before this one has already formed (for every segment but
        // the last): copy it transposed instead of scanning K again.
        const float* A = fmaps + (u * (nseg - 1) + s) * 2 * kD * kD;
        float* Lm = gmaps + ((u * (nseg - 1) + (nseg - 1 - s)) * 2) * kD * kD;
        for (int e = threadIdx.x; e < kD * kD; e += kThreads)
            Lm[(e % kD) * kD + e / kD] = A[e];
        return;
    }
    const int h = static_cast<int>(u % H);
    const float et = eta[h];
    const int seg_chunks = seg_len / kB;
    const int c0 = s * seg_chunks;
    const int c1 = min((T + kB - 1) / kB, c0 + seg_chunks);
    const int64_t off = u * static_cast<int64_t>(T) * kD;
    const int64_t chain_bytes = static_cast<int64_t>(T) * kD * 2;
    const __amdgpu_buffer_rsrc_t r_q = buffer_rsrc(Q + off, chain_bytes);
    const __amdgpu_buffer_rsrc_t r_k = buffer_rsrc(K + off, chain_bytes);
    const __amdgpu_buffer_rsrc_t r_v = buffer_rsrc(V + off, kGMap ? 0 : chain_bytes);
    const __amdgpu_buffer_rsrc_t r_dy = buffer_rsrc(dY + off, chain_bytes);
    const __amdgpu_buffer_rsrc_t r_dq = buffer_rsrc(dQ + off, kGMap ? 0 : chain_bytes);
    const __amdgpu_buffer_rsrc_t r_dk = buffer_rsrc(dK + off, kGMap ? 0 : chain_bytes);
    const __amdgpu_buffer_rsrc_t r_dv = buffer_rsrc(dV + off, kGMap ? 0 : chain_bytes);
    // this segment's update operands E' in the workspace: [chunk][thread] x 8 bytes
    uint16_t* st = states + (u * nseg + s) * static_cast<int64_t>(seg_chunks) * kThreads * 4;
    const __amdgpu_buffer_rsrc_t r_st =
        buffer_rsrc(st, kGMap ? 0 : static_cast<int64_t>(seg_chunks) * kThreads * 8);
    const bool use_dy = !kGMap || half == 1;     // uniform per workgroup
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // staging of the 16 x 64 tiles: thread tid moves 8 bytes of row tid / 16
    const int srow = tid >> 4;
    const int scol = 4 * (tid & 15);
    const int sbyte = swz(srow, scol >> 3) + 8 * (tid & 1);

    // prologue state of this staging thread: gamma, beta of its 4 columns,
    // the normalised rows and 1/std of the chunk last staged (its epilogue
    // runs before the next chunk is staged), and the gamma, beta gradients
    const bool use_tok = kPro && pro.eta_tok != nullptr;
    const bool ln_q = kPro && pro.ln_q != nullptr;
    const bool ln_k = kPro && pro.ln_k != nullptr;
    const bool a_on = !kPro || !pro.read_start;      // uniform: the tril(Q K^T) term
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
        buffer_rsrc(use_tok ? pro.eta_tok + u * static_cast<int64_t>(T) : eta,
                   use_tok ? static_cast<int64_t>(T) * 4 : 0);
    const __amdgpu_buffer_rsrc_t r_deta =
        buffer_rsrc(use_tok && !kGMap ? deta_tok + u * static_cast<int64_t>(T) : eta,
                   use_tok && !kGMap ? static_cast<int64_t>(T) * 4 : 0);
    // LayerNorm of a staged row segment, back to bf16; keeps xh and 1/std
    auto norm = [&](u32x2 x, const float (&gm)[4], const float (&bt)[4], bool valid,
                    float (&xh)[4], float& rstd) {
        float f[4];
        unpack4(x, f);
        layernorm_row_keep<16, 4>(f, pro.ln_eps, valid, xh, rstd);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            f[e] = valid ? xh[e] * gm[e] + bt[e] : 0.f;
        return u32x2{cvt2(f[0], f[1]), cvt2(f[2], f[3])};
    };
    auto load_stage = [&](Stage& x, int chunk, bool qdy, bool wst, bool with_v = true) {
        const int t = chunk * kB + srow;
        const int eb = (t * kD + scol) * 2;
        x.ok = t < T;
        if constexpr (kPro) {
            const float tok = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_eta, t * 4, 0, 0));
            x.eta = use_tok ? tok : (x.ok ? et : 0.f);
        }
        x.k = __builtin_amdgcn_raw_buffer_load_b64(r_k, eb, 0, 0);
        if (qdy) {
            x.q = __builtin_amdgcn_raw_buffer_load_b64(r_q, eb, 0, 0);
            x.dy = __builtin_amdgcn_raw_buffer_load_b64(r_dy, eb, 0, 0);
        }
        if (!kGMap && with_v) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                x.v[r] = __builtin_amdgcn_raw_buffer_load_b32(
                    r_v, ((chunk * kB + 4 * g + r) * kD + (col & ~1)) * 2, 0, 0);
        }
        if (wst) {
            // chunk c0 - 1 (loaded ahead of the first chunk) falls outside:
            // zeros; the segment's last chunk has none (unused)
            x.e = __builtin_amdgcn_raw_buffer_load_b64(r_st, ((chunk - c0) * kThreads + tid) * 8, 0, 0);
        }
    };
    // (with the prologue: LayerNorm first, and the rows' step sizes)
    auto store_stage = [&](const Stage& x, int slot, bool qdy) {
        unsigned char* sl = lds + slot * kSlotBytes;
        u32x2 kx = x.k, qx = x.q;
        if constexpr (kPro) {
            if (ln_k)
                kx = norm(x.k, gmk, btk, x.ok, xk, rk);
            if (qdy && ln_q)
                qx = norm(x.q, gmq, btq, x.ok, xq, rq);
            if ((tid & 15) == 0)
                reinterpret_cast<float*>(lds + L::kEta)[slot * kB + srow] = x.eta;
        }
        *reinterpret_cast<u32x2*>(sl + kSlotK + sbyte) = kx;
        if (qdy) {
            *reinterpret_cast<u32x2*>(sl + kSlotQ + sbyte) = qx;
            *reinterpret_cast<u32x2*>(sl + kSlotDY + sbyte) = x.dy;
        }
    };
    // step sizes of rows 4g .. 4g + 3 of a slot (the head's without the prologue)
    auto rows_eta = [&](int slot) {
        if constexpr (kPro)
            return *reinterpret_cast<const f32x4*>(lds + L::kEta + 4 * (slot * kB + 4 * g));
        else
            return f32x4{et, et, et, et};
    };
    auto vneg = [&](const uint32_t (&v)[4]) {
        f32x4 r;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            r[q] = -__uint_as_float((col & 1) ? (v[q] & 0xffff0000u) : (v[q] << 16));
        return r;
    };

    // ---------------- sweep 1: chunk-start states of the segment ----------------
    f32x4 Wacc[4];               // W[rho(mt, 4g + r)][col]; after sweep 1 W of chunk c1 - 1
    if (!kGMap && c1 > c0) {
        {
            const float* w0 = nseg > 1 ? wstart + (u * nseg + s) * kD * kD
                                       : W0 + (w0_per_batch ? u : h) * kD * kD;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Wacc[mt][r] = w0[rho(mt, 4 * g + r) * kD + col];
        }
        // The chunks ahead in two rings of kAhead register sets: K of chunk
        // ch + 1 in kring[(ch - c0) % kAhead] (written to LDS at chunk ch),
        // V of chunk ch in vring[(ch - c0) % kAhead] (used at chunk ch, each
        // entry in place, so no register copy waits for a load in flight);
        // the loop runs in rounds of kAhead chunks to keep the ring indices
        // static, and a scheduling barrier closes each step
        constexpr int kAhead = 4;
        Stage kring[kAhead];
        uint32_t vring[kAhead][4];
        auto load_v = [&](uint32_t (&v)[4], int chunk) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v[r] = __builtin_amdgcn_raw_buffer_load_b32(
                    r_v, ((chunk * kB + 4 * g + r) * kD + (col & ~1)) * 2, 0, 0);
        };
        {
            Stage first;
            load_stage(first, c0, false, false, false);
            store_stage(first, 0, false);
        }
#pragma unroll
        for (int q = 0; q < kAhead; ++q) {
            load_v(vring[q], c0 + q);
            load_stage(kring[q], c0 + 1 + q, false, false, false);
        }
        __syncthreads();
        // (`last`: the segment's last chunk, whose W stays in the registers
        // for sweep 2; a constant false in the full rounds)
        auto sweep1_step = [&](int ch, Stage& knext, uint32_t (&vc)[4], bool last) {
            if (last)
                return;
            // W_c^T row col: 16 bytes at i = 8g .. and 32 + 8g ..
            const bf16x8 b0 = pack8(Wacc[0], Wacc[1]);
            const bf16x8 b1 = pack8(Wacc[2], Wacc[3]);
            const unsigned char* sl = lds + ((ch - c0) & 1) * kSlotBytes;
            // E = K W_J - V, W += K^T (-eta E); E' = -eta E goes to the workspace
            f32x4 R = mfma32(row8(sl + kSlotK, c, g), b0, vneg(vc));
            R = mfma32(row8(sl + kSlotK, c, 4 + g), b1, R);
            const bf16x4 eb = pack4(-(rows_eta((ch - c0) & 1) * R));
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, eb), r_st,
                                                  ((ch - c0) * kThreads + tid) * 8, 0, 0);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                Wacc[mt] = mfma16(col4_rho(sl + kSlotK, 4 * g, mt, c), eb, Wacc[mt]);
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
        // the operands just stored are read back below (by the threads that wrote them)
        __threadfence();
        __syncthreads();
    }

    // ---------------- sweep 2: reverse over the chunks of the segment ----------------
    f32x4 Gacc[4];               // G[rho(mt, 4g + r)][col]
    if (kGMap) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Gacc[mt][r] = half == 0 && rho(mt, 4 * g + r) == col ? 1.f : 0.f;
    } else {
        const float* g1 = nseg > 1 ? gend + (u * nseg + (nseg - 1 - s)) * kD * kD
                                   : dW_out + u * kD * kD;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Gacc[mt][r] = g1[rho(mt, 4 * g + r) * kD + col];
    }
    float deta_acc = 0.f;

    uint32_t vcur[4] = {0, 0, 0, 0};
    u32x2 ecur = {0, 0};         // E' of the chunk in hand (none for the last)
    if (c1 > c0) {
        Stage nx;
        load_stage(nx, c1 - 1, use_dy, false);
        store_stage(nx, 0, use_dy);
        if (!kGMap) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vcur[r] = nx.v[r];
        }
        __syncthreads();
    }
    for (int ch = c1 - 1; ch >= c0; --ch) {
        const int slot = (c1 - 1 - ch) & 1;
        const unsigned char* sl = lds + slot * kSlotBytes;
        Stage nx;
        // (unconditional, so the loads keep exact wait counts: at the first
        // chunk it reads chunk c0 - 1, unused, zeros where it is outside)
        load_stage(nx, ch - 1, use_dy, !kGMap);

        // ---- phase A: columns J = w ----
        const bf16x8 ka0 = row8(sl + kSlotK, c, g);
        const bf16x8 ka1 = row8(sl + kSlotK, c, 4 + g);
        const bf16x8 gb0 = pack8(Gacc[0], Gacc[1]);       // G'_J as a B operand
        const bf16x8 gb1 = pack8(Gacc[2], Gacc[3]);
        f32x4 E = zero;
        if (!kGMap) {
            // W_c from W_{c+1}: undo sweep 1's update of this chunk (uniform)
            if (ch < c1 - 1) {
                const bf16x4 en = __builtin_bit_cast(bf16x4, ecur ^ u32x2{0x80008000u, 0x80008000u});
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    Wacc[mt] = mfma16(col4_rho(sl + kSlotK, 4 * g, mt, c), en, Wacc[mt]);
            }
            // W_c^T row col (i = 8g .. and 32 + 8g ..) for this wave's E and,
            // through LDS, for every wave's phase B
            const bf16x8 b0 = pack8(Wacc[0], Wacc[1]);
            const bf16x8 b1 = pack8(Wacc[2], Wacc[3]);
            *reinterpret_cast<bf16x8*>(lds + kOffW + swz(col, g)) = b0;
            *reinterpret_cast<bf16x8*>(lds + kOffW + swz(col, 4 + g)) = b1;
            E = mfma32(ka0, b0, vneg(vcur));
            E = mfma32(ka1, b1, E);
        }
        // P = A^T dY_J + K G'_J  (A = tril(Q K^T); S holds S[t = 4g + r][s = c])
        f32x4 P1 = zero;
        bf16x4 dyt = {};
        if (use_dy) {
            dyt = col4(sl + kSlotDY, 4 * g, 16 * w, c);  // dY[4g + r][col]
            if (a_on) {
                f32x4 S = mfma32(row8(sl + kSlotQ, c, g), ka0, zero);
                S = mfma32(row8(sl + kSlotQ, c, 4 + g), ka1, S);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[r] = c <= 4 * g + r ? S[r] : 0.f;
                P1 = mfma16(pack4(S), dyt, zero);
            }
        }
        f32x4 P2 = mfma32(ka0, gb0, zero);
        P2 = mfma32(ka1, gb1, P2);
        const f32x4 P = P1 + P2;
        const f32x4 er = rows_eta(slot);                  // eta of rows 4g + r
        const f32x4 dE = -(er * P);
        if (!kGMap) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (kPro) {
                    if (use_tok) {
                        // -<P_t, E_t> over this wave's 16 columns
                        const float pe = group_sum<16>(P[r] * E[r]);
                        if (c == 0)
                            reinterpret_cast<float*>(lds + L::kDeta)[w * kB + 4 * g + r] = pe;
                    } else {
                        deta_acc -= P[r] * E[r];
                    }
                } else {
                    deta_acc -= P[r] * E[r];
                }
                *reinterpret_cast<__bf16*>(lds + kOffE + swz_elem(4 * g + r, col)) = static_cast<__bf16>(E[r]);
                *reinterpret_cast<__bf16*>(lds + kOffP + swz_elem(4 * g + r, col)) = static_cast<__bf16>(P[r]);
            }
            // G'^T row col: i = 8g .. and 32 + 8g ..
            *reinterpret_cast<bf16x8*>(lds + kOffG + swz(col, g)) = gb0;
            *reinterpret_cast<bf16x8*>(lds + kOffG + swz(col, 4 + g)) = gb1;
        }
        // G = G' + Q^T dY_J + K^T dE  (over the 16 tokens; A in rho order)
        const bf16x4 deb = pack4(dE);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f32x4 acc = Gacc[mt];
            if (use_dy)
                acc = mfma16(col4_rho(sl + kSlotQ, 4 * g, mt, c), dyt, acc);
            Gacc[mt] = mfma16(col4_rho(sl + kSlotK, 4 * g, mt, c), deb, acc);
        }

        if (!kGMap) {
            __syncthreads();
            // ---- phase B: input dims I = w ----
            // W[16 w + c][32 q + 8g ..], written by the four waves before the barrier
            bf16x8 wb[2];
#pragma unroll
            for (int q = 0; q < 2; ++q)
                wb[q] = join(col4(lds + kOffW, 32 * q + 8 * g, 16 * w, c),
                             col4(lds + kOffW, 32 * q + 8 * g + 4, 16 * w, c));
            const bf16x8 ya0 = row8(sl + kSlotDY, c, g), ya1 = row8(sl + kSlotDY, c, 4 + g);
            const bf16x8 ea0 = row8(lds + kOffE, c, g), ea1 = row8(lds + kOffE, c, 4 + g);
            // dA[t = 4g + r][s = c] and dA^T[s = 4g + r][t = c], masked and scaled
            f32x4 dA = zero, dAT = zero;
            if (a_on) {
                dA = mfma32(ya0, ea0, zero);
                dA = mfma32(ya1, ea1, dA);
                dAT = mfma32(ea0, ya0, zero);
                dAT = mfma32(ea1, ya1, dAT);
                // dA[t][s] scales by eta_s (s = c), dA^T[s][t] by eta_s (s = 4g + r)
                const float ec = kPro ? reinterpret_cast<const float*>(lds + L::kEta)[slot * kB + c] : et;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dA[r] = c <= 4 * g + r ? -ec * dA[r] : 0.f;
                    dAT[r] = 4 * g + r <= c ? -er[r] * dAT[r] : 0.f;
                }
            }
            // dQ_I = dY W[I, :]^T + dA K_I
            f32x4 q1 = mfma32(ya0, wb[0], zero);
            q1 = mfma32(ya1, wb[1], q1);
            f32x4 dq = q1;
            if (a_on)
                dq += mfma16(pack4(dAT), col4(sl + kSlotK, 4 * g, 16 * w, c), zero);
            // dK_I = -eta (P W[I, :]^T + E G'[I, :]^T) + dA^T Q_I
            bf16x8 gt[2];
#pragma unroll
            for (int q = 0; q < 2; ++q)
                gt[q] = join(col4(lds + kOffG, 32 * q + 8 * g, 16 * w, c),
                             col4(lds + kOffG, 32 * q + 8 * g + 4, 16 * w, c));
            f32x4 k1 = mfma32(row8(lds + kOffP, c, g), wb[0], zero);
            k1 = mfma32(row8(lds + kOffP, c, 4 + g), wb[1], k1);
            k1 = mfma32(ea0, gt[0], k1);
            k1 = mfma32(ea1, gt[1], k1);
            f32x4 dk = -(er * k1);
            if (a_on)
                dk += mfma16(pack4(dA), col4(sl + kSlotQ, 4 * g, 16 * w, c), zero);

            // rows t = 16 ch + 4g + r, column 16 w + c; dV = eta P (this wave's
            // columns from phase A)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int eb = ((ch * kB + 4 * g + r) * kD + col) * 2;    // past T: dropped
                if constexpr (!kPro) {
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(dq[r]), r_dq, eb, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(dk[r]), r_dk, eb, 0, 0);
                }
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(er[r] * P[r]), r_dv, eb, 0, 0);
            }
            if constexpr (kPro) {
                // the gradients of the normalised rows go to the staging
                // threads for the LayerNorm backward
                float* tq = reinterpret_cast<float*>(lds + L::kDQ);
                float* tk = reinterpret_cast<float*>(lds + L::kDK);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    tq[(4 * g + r) * kFP + col] = dq[r];
                    tk[(4 * g + r) * kFP + col] = dk[r];
                }
                __syncthreads();
                float gq[4], gk[4];
                {
                    const f32x4 a = *reinterpret_cast<const f32x4*>(tq + srow * kFP + scol);
                    const f32x4 b = *reinterpret_cast<const f32x4*>(tk + srow * kFP + scol);
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
                const int eb = (t * kD + scol) * 2;                     // past T: dropped
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{cvt2(gq[0], gq[1]), cvt2(gq[2], gq[3])},
                                                      r_dq, eb, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{cvt2(gk[0], gk[1]), cvt2(gk[2], gk[3])},
                                                      r_dk, eb, 0, 0);
                if (use_tok) {
                    // the row's 16 lanes store the same sum (no branch)
                    const float* pd = reinterpret_cast<const float*>(lds + L::kDeta);
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
                ecur = nx.e;
            }
        }
        __syncthreads();
    }

    if (kGMap) {
        float* out = gmaps + ((u * (nseg - 1) + (nseg - 1 - s)) * 2 + half) * kD * kD;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                out[rho(mt, 4 * g + r) * kD + col] = Gacc[mt][r];
        return;
    }
    if (s == 0) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dW0_chain[u * kD * kD + rho(mt, 4 * g + r) * kD + col] = Gacc[mt][r];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        deta_acc += __shfl_xor(deta_acc, m);
    float* red = reinterpret_cast<float*>(lds + kOffRed);
    if (lane == 0)
        red[w] = deta_acc;
    if constexpr (kPro) {
        // gamma, beta gradients: over the 4 rows of the wave (lanes 16 apart),
        // then over the waves; out[a][col], a = gamma_q, beta_q, gamma_k, beta_k
        float* lr = reinterpret_cast<float*>(lds + L::kDQ);    // [4 waves][4][64]
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
        const float x = (lr[tid] + lr[256 + tid]) + (lr[512 + tid] + lr[768 + tid]);
        dln_chain[(u * nseg + s) * (kDlnRows * kD) + tid] = x;
    } else {
        __syncthreads();
    }
    if (tid == 0)
        deta_chain[u * nseg + s] = (red[0] + red[1]) + (red[2] + red[3]);
}

template <bool kGMap, bool kPro>
void launch_bf16(const LinearBwdArgs& a, const SegmentPlan& p, const BwdBuffers& b, dim3 grid)
{
    hipLaunchKernelGGL((linear_backward_bf16_kernel<kGMap, kPro>), grid, dim3(kThreads),
                       kGMap ? Lay<kPro>::kGMapBytes : Lay<kPro>::kBytes, a.stream,
                       static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                       static_cast<const uint16_t*>(a.V), a.W0, a.w0_per_batch, a.eta,
                       static_cast<int>(a.H), static_cast<int>(a.T), a.B * a.H,
                       static_cast<int>(p.seg_len), p.nseg, b.wstart, b.gend,
                       static_cast<const uint16_t*>(a.dY), a.dW_out, static_cast<uint16_t*>(a.dQ),
                       static_cast<uint16_t*>(a.dK), static_cast<uint16_t*>(a.dV), b.dw_chain,
                       b.deta_chain, reinterpret_cast<uint16_t*>(b.states), b.gmaps, a.pro,
                       a.deta_tok, b.dln_chain, b.maps);
}

}  // namespace

hipError_t launch_linear_backward_bf16(const LinearBwdArgs& a, const SegmentPlan& p, bool gmap,
                                       const BwdBuffers& b, dim3 grid)
{
    const bool pro = a.pro.active();
    if (gmap)
        pro ? launch_bf16<true, true>(a, p, b, grid) : launch_bf16<true, false>(a, p, b, grid);
    else
        pro ? launch_bf16<false, true>(a, p, b, grid) : launch_bf16<false, false>(a, p, b, grid);
    return hipGetLastError();
}

}  // namespace ttt
