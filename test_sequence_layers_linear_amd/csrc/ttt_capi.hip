// ttt_capi.hip -- the C ABI declared in include/ttt.h: argument validation,
// kernel selection and launch on the caller's stream.  Validation happens
// before any HIP call, so every error path is reachable without a GPU.
#include "ttt.h"
#include "ttt_internal.h"

#include <stdint.h>

#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

namespace {

using ttt::LinearArgs;
using ttt::MlpArgs;
using ttt::DecodeArgs;

constexpr int kAbiVersion = (1 << 16) | 2;

bool valid_dtype(int dt) { return dt == TTT_F32 || dt == TTT_BF16; }
size_t elem_bytes(int dt) { return dt == TTT_F32 ? 4 : 2; }

// a*b*c*... with overflow detection (all factors >= 0)
bool mul_ok(int64_t& acc, int64_t x)
{
    int64_t r;
    if (__builtin_mul_overflow(acc, x, &r)) return false;
    acc = r;
    return true;
}

struct Range {
    const void* p;
    int64_t bytes;
};

bool overlap(const Range& a, const Range& b)
{
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

bool d_supported(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// largest grid.x the launchers use
constexpr int64_t kMaxUnits = 0x7fffffff;

int hip_status(hipError_t e) { return e == hipSuccess ? TTT_OK : TTT_ERR_HIP; }

// Compute units of the current device (cached per device).
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Segment count for a chain-parallel scan of `units` chains of T tokens.
// Each launch of the split runs all its workgroups at once, one per CU (more
// would queue or share CUs and stretch the slowest ones), so S is limited to
// what fits; within that it minimises
//   ceil(chunks / S) (map + fwd) + (S - 1) apply + launch
// against the unsplit chunks * fwd (costs measured on MI355X).
// TTT_LINEAR_SEGMENTS=S (1 <= S <= kMaxSegments) forces S segments (at least
// one chunk each), for tests and tuning.
ttt::SegmentPlan plan_segments(int64_t units, int64_t T, int chunk, const ttt::SegmentCosts& cost)
{
    ttt::SegmentPlan p;
    p.seg_len = T;
    const int64_t chunks = (T + chunk - 1) / chunk;
    if (const char* env = getenv("TTT_LINEAR_SEGMENTS")) {
        const long S = std::min<long>(strtol(env, nullptr, 10), ttt::kMaxSegments);
        if (S >= 1 && chunks > 0) {
            p.seg_len = ((chunks + S - 1) / S) * chunk;
            p.nseg = static_cast<int>((T + p.seg_len - 1) / p.seg_len);
            return p;
        }
    }
    const int64_t cus = device_cus();
    const int64_t scan_blocks = units * cost.scan_blocks_per_segment;
    if (cus <= 0 || 2 * scan_blocks > cus || chunks < 4) return p;
    double best = static_cast<double>(chunks) * cost.fwd;
    int best_s = 1;
    for (int S = 2; S <= ttt::kMaxSegments; ++S) {
        if (scan_blocks * S > cus ||
            units * (S - 1) * cost.map_blocks_per_segment > cost.map_blocks_per_cu * cus)
            break;
        const int64_t per = (chunks + S - 1) / S;
        if (per < 2) break;
        const double t = per * (cost.map + cost.fwd) + (S - 1) * cost.apply + cost.launch;
        if (t < best) { best = t; best_s = S; }
    }
    if (best_s > 1) {
        p.seg_len = ((chunks + best_s - 1) / best_s) * chunk;
        p.nseg = static_cast<int>((T + p.seg_len - 1) / p.seg_len);
    }
    return p;
}

// Segment count for the backward of a TTT-Linear scan: each segment pays
// its chunks' forward map, cotangent map and backward, and the two
// compositions (S - 1) steps each, plus four extra launches.  Up to
// max_per_cu segment-backward workgroups share a CU, each slowed by `share`
// per extra workgroup per CU; the maps launches may hold maps_per_cu per CU.
// TTT_LINEAR_BWD_SEGMENTS=S forces S segments.
ttt::SegmentPlan plan_backward(int64_t units, int64_t T, int chunk, const ttt::BwdCosts& cost)
{
    ttt::SegmentPlan p;
    p.seg_len = T;
    const int64_t chunks = (T + chunk - 1) / chunk;
    if (const char* env = getenv("TTT_LINEAR_BWD_SEGMENTS")) {
        const long S = std::min<long>(strtol(env, nullptr, 10), ttt::kMaxSegments);
        if (S >= 1 && chunks > 0) {
            p.seg_len = ((chunks + S - 1) / S) * chunk;
            p.nseg = static_cast<int>((T + p.seg_len - 1) / p.seg_len);
            return p;
        }
    }
    const int64_t cus = device_cus();
    if (cus <= 0 || 2 * units > cost.max_per_cu * cus || chunks < 4) return p;
    const int map_blocks = std::max(2, cost.fmap_blocks_per_segment);
    double best = static_cast<double>(chunks) * cost.bwd;
    int best_s = 1;
    for (int S = 2; S <= ttt::kMaxSegments; ++S) {
        if (units * S > cost.max_per_cu * cus || units * (S - 1) * map_blocks > cost.maps_per_cu * cus)
            break;
        const int64_t per = (chunks + S - 1) / S;
        if (per < 2) break;
        const double load = std::max(1.0, static_cast<double>(units * S) / static_cast<double>(cus));
        const double t = per * (cost.bwd * (1.0 + cost.share * (load - 1.0)) + cost.fmap + cost.gmap) +
                         2.0 * (S - 1) * cost.apply + cost.launch;
        if (t < best) { best = t; best_s = S; }
    }
    if (best_s > 1) {
        p.seg_len = ((chunks + best_s - 1) / best_s) * chunk;
        p.nseg = static_cast<int>((T + p.seg_len - 1) / p.seg_len);
    }
    return p;
}

// Workspace for the segment maps: one device buffer per (device, stream),
// grown on demand and kept until the process ends.  Calls on one stream are
// ordered by the stream, so they can share its buffer; calls on different
// streams get different buffers.  Before a buffer is replaced by a larger one
// its stream is synchronised, so no enqueued kernel still uses it.
hipError_t workspace_get(void** ptr, size_t bytes, hipStream_t stream)
{
    struct Entry {
        int dev;
        hipStream_t stream;
        void* p;
        size_t bytes;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    Entry* hit = nullptr;
    for (Entry& x : cache)
        if (x.dev == dev && x.stream == stream) hit = &x;
    if (hit && hit->bytes >= bytes) {
        *ptr = hit->p;
        return hipSuccess;
    }
    if (hit) {
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return e;
        e = hipFree(hit->p);
        hit->p = nullptr;
        hit->bytes = 0;
        if (e != hipSuccess) return e;
    }
    void* p = nullptr;
    e = hipMalloc(&p, bytes);
    if (e != hipSuccess) return e;
    if (hit) {
        hit->p = p;
        hit->bytes = bytes;
    } else {
        cache.push_back(Entry{dev, stream, p, bytes});
    }
    *ptr = p;
    return hipSuccess;
}

// fp32 scans split each chain's columns over 4 workgroups while those fit the
// CUs (fewer chains than a quarter of the CUs); with more chains the GPU is
// already full and the one-workgroup kernel does the same MFMA work with less
// traffic.  TTT_LINEAR_F32_COLS=0 turns the split off.
bool use_cols_f32(const LinearArgs& a)
{
    if (!ttt::linear_cols_f32_supports(a)) return false;
    if (const char* env = getenv("TTT_LINEAR_F32_COLS"))
        if (strtol(env, nullptr, 10) == 0) return false;
    const int64_t cus = device_cus();
    return cus > 0 && a.B * a.H * ttt::kColsSlices <= cus;
}

// Runs a segmented MFMA linear scan: workspace for the maps and the segment
// start states, then the launches.  The start states (including the copy of
// W0 for the first segment) are complete before any segment writes W_out, so
// W_out may overwrite W0.
int run_linear_segmented(LinearArgs a, ttt::SegmentPlan p,
                         hipError_t (*launch)(const LinearArgs&, const ttt::SegmentPlan&))
{
    if (p.nseg <= 1) return hip_status(launch(a, p));
    const int64_t units = a.B * a.H;
    const size_t state = static_cast<size_t>(a.d) * a.d * sizeof(float);
    const size_t map_bytes = static_cast<size_t>(units) * (p.nseg - 1) * 2 * state;
    const size_t start_bytes = static_cast<size_t>(units) * p.nseg * state;
    void* ws = nullptr;
    if (workspace_get(&ws, map_bytes + start_bytes, a.stream) != hipSuccess) return TTT_ERR_HIP;
    p.maps = static_cast<float*>(ws);
    p.wstart = p.maps + map_bytes / sizeof(float);
    return hip_status(launch(a, p));
}

}  // namespace

extern "C" {

int ttt_abi_version(void) { return kAbiVersion; }

const char* ttt_status_string(int status)
{
    switch (status) {
    case TTT_OK: return "ok";
    case TTT_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size, b < 1, bad flag or overlapping buffers)";
    case TTT_ERR_UNSUPPORTED: return "unsupported shape or dtype (d, m, b, dtype, or on-chip memory the shape needs)";
    case TTT_ERR_HIP: return "a HIP call or kernel launch failed";
    default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// ttt_linear_forward with an optional input prologue (pro.active(): d = 64,
// b = 16 only).
int linear_forward_impl(const void* Q, const void* K, const void* V, int qkv_dtype,
                        const float* W0, int w0_per_batch, const float* eta,
                        int64_t B, int64_t H, int64_t T, int d, int b,
                        void* Y, float* W_out, void* stream, const ttt::Prologue& pro)
{
    if (B < 0 || H < 0 || T < 0 || b < 1 || (w0_per_batch != 0 && w0_per_batch != 1))
        return TTT_ERR_INVALID_ARG;
    if (!valid_dtype(qkv_dtype) || !d_supported(d) || b > 64)
        return TTT_ERR_UNSUPPORTED;
    int64_t units = B;
    if (!mul_ok(units, H) || units > kMaxUnits) return TTT_ERR_UNSUPPORTED;
    if (units == 0) return TTT_OK;
    int64_t n_qkv = units;
    if (!mul_ok(n_qkv, T) || !mul_ok(n_qkv, d) || !mul_ok(n_qkv, 4)) return TTT_ERR_UNSUPPORTED;
    n_qkv = n_qkv / 4 * static_cast<int64_t>(elem_bytes(qkv_dtype));
    const int64_t n_state = static_cast<int64_t>(d) * d * 4;
    if (!W0 || !eta || !W_out) return TTT_ERR_INVALID_ARG;
    if (T > 0 && (!Q || !K || !V || !Y)) return TTT_ERR_INVALID_ARG;

    const Range rQ{Q, T ? n_qkv : 0}, rK{K, T ? n_qkv : 0}, rV{V, T ? n_qkv : 0};
    const Range rY{Y, T ? n_qkv : 0};
    const Range rW0{W0, (w0_per_batch ? units : H) * n_state};
    const Range rWo{W_out, units * n_state}, rEta{eta, H * 4};
    for (const Range& in : {rQ, rK, rV, rW0, rEta, rWo})
        if (overlap(rY, in)) return TTT_ERR_INVALID_ARG;
    for (const Range& in : {rQ, rK, rV, rEta})
        if (overlap(rWo, in)) return TTT_ERR_INVALID_ARG;
    if (overlap(rWo, rW0) && !(w0_per_batch && static_cast<const void*>(W_out) == W0))
        return TTT_ERR_INVALID_ARG;
    if (pro.active()) {
        const Range rTok{pro.eta_tok, pro.eta_tok ? units * T * 4 : 0};
        const Range rLq{pro.ln_q, pro.ln_q ? H * 2 * d * 4 : 0}, rLk{pro.ln_k, pro.ln_k ? H * 2 * d * 4 : 0};
        for (const Range& in : {rTok, rLq, rLk})
            if (overlap(rY, in) || overlap(rWo, in)) return TTT_ERR_INVALID_ARG;
    }

    LinearArgs a{Q, K, V, qkv_dtype, W0, w0_per_batch, eta, B, H, T, d, b,
                 Y, W_out, static_cast<hipStream_t>(stream)};
    a.pro = pro;
    if (pro.active() && !ttt::linear_mfma_supports(a) && !ttt::linear_mfma_f32_supports(a))
        return TTT_ERR_UNSUPPORTED;
    if (ttt::linear_mfma_supports(a))
        return run_linear_segmented(a, plan_segments(units, T, b, ttt::kLinearBf16Costs),
                                    ttt::launch_linear_mfma);
    if (use_cols_f32(a))
        return run_linear_segmented(a, plan_segments(units, T, b, ttt::kLinearF32ColsCosts),
                                    ttt::launch_linear_cols_f32);
    if (ttt::linear_mfma_f32_supports(a))
        return run_linear_segmented(a, plan_segments(units, T, b, ttt::kLinearF32Costs),
                                    ttt::launch_linear_mfma_f32);
    if (ttt::linear_generic_lds_bytes(d, b) > static_cast<size_t>(ttt::kMaxLdsBytes))
        return TTT_ERR_UNSUPPORTED;
    return hip_status(ttt::launch_linear_generic(a));
}


}  // namespace

extern "C" {

int ttt_linear_forward(const void* Q, const void* K, const void* V, int qkv_dtype,
                       const float* W0, int w0_per_batch, const float* eta,
                       int64_t B, int64_t H, int64_t T, int d, int b,
                       void* Y, float* W_out, void* stream)
{
    return linear_forward_impl(Q, K, V, qkv_dtype, W0, w0_per_batch, eta, B, H, T, d, b, Y, W_out,
                               stream, ttt::Prologue{});
}

int ttt_linear_forward_ex(const void* Q, const void* K, const void* V, int qkv_dtype,
                          const float* W0, int w0_per_batch, const float* eta,
                          const float* eta_tok, const float* ln_q, const float* ln_k, float ln_eps,
                          int read_mode, int64_t B, int64_t H, int64_t T, int d, int b,
                          void* Y, float* W_out, void* stream)
{
    if ((ln_q || ln_k) && !(ln_eps > 0.0f && ln_eps < 1e30f))
        return TTT_ERR_INVALID_ARG;
    if (read_mode != 0 && read_mode != 1)
        return TTT_ERR_INVALID_ARG;
    ttt::Prologue pro;
    pro.eta_tok = eta_tok;
    pro.ln_q = ln_q;
    pro.ln_k = ln_k;
    pro.ln_eps = ln_eps;
    pro.read_start = read_mode;
    if (pro.active() && B * H > 0 && T > 0 && (d != 64 || b != 16))
        return TTT_ERR_UNSUPPORTED;
    return linear_forward_impl(Q, K, V, qkv_dtype, W0, w0_per_batch, eta, B, H, T, d, b, Y, W_out,
                               stream, pro);
}

int ttt_linear_segments(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype)
{
    if (B < 0 || H < 0 || T < 0 || b < 1) return TTT_ERR_INVALID_ARG;
    if (!valid_dtype(qkv_dtype) || !d_supported(d) || b > 64) return TTT_ERR_UNSUPPORTED;
    int64_t units = B;
    if (!mul_ok(units, H) || units > kMaxUnits) return TTT_ERR_UNSUPPORTED;
    LinearArgs a{nullptr, nullptr, nullptr, qkv_dtype, nullptr, 0, nullptr, B, H, T, d, b,
                 nullptr, nullptr, nullptr};
    if (units == 0 || T == 0) return 1;
    if (ttt::linear_mfma_supports(a)) return plan_segments(units, T, b, ttt::kLinearBf16Costs).nseg;
    if (use_cols_f32(a)) return plan_segments(units, T, b, ttt::kLinearF32ColsCosts).nseg;
    if (ttt::linear_mfma_f32_supports(a)) return plan_segments(units, T, b, ttt::kLinearF32Costs).nseg;
    return 1;
}

}  // extern "C"

namespace {

int linear_backward_impl(const void* Q, const void* K, const void* V, int qkv_dtype,
                         const float* W0, int w0_per_batch, const float* eta,
                         int64_t B, int64_t H, int64_t T, int d, int b,
                         const void* dY, const float* dW_out,
                         void* dQ, void* dK, void* dV, float* dW0, float* deta,
                         const ttt::Prologue& pro, float* deta_tok, float* dln_q, float* dln_k,
                         void* stream)
{
    if (B < 0 || H < 0 || T < 0 || b < 1 || (w0_per_batch != 0 && w0_per_batch != 1))
        return TTT_ERR_INVALID_ARG;
    if (!valid_dtype(qkv_dtype) || d != 64 || b != 16)
        return TTT_ERR_UNSUPPORTED;
    int64_t units = B;
    if (!mul_ok(units, H) || units > kMaxUnits) return TTT_ERR_UNSUPPORTED;
    int64_t n_qkv = units;
    if (!mul_ok(n_qkv, T) || !mul_ok(n_qkv, d) || !mul_ok(n_qkv, 4)) return TTT_ERR_UNSUPPORTED;
    n_qkv = n_qkv / 4 * static_cast<int64_t>(elem_bytes(qkv_dtype));
    const int64_t n_state = static_cast<int64_t>(d) * d * 4;
    if (H > 0 && (!dW0 || !deta)) return TTT_ERR_INVALID_ARG;
    if (units > 0 && (!W0 || !eta || !dW_out)) return TTT_ERR_INVALID_ARG;
    if (units > 0 && T > 0 && (!Q || !K || !V || !dY || !dQ || !dK || !dV)) return TTT_ERR_INVALID_ARG;
    // each prologue input comes with its gradient output
    if ((pro.eta_tok != nullptr) != (deta_tok != nullptr) || (pro.ln_q != nullptr) != (dln_q != nullptr) ||
        (pro.ln_k != nullptr) != (dln_k != nullptr))
        return TTT_ERR_INVALID_ARG;
    if (H == 0) return TTT_OK;

    const int64_t nq = units > 0 && T > 0 ? n_qkv : 0;
    const int64_t ntok = units > 0 && T > 0 ? units * T * 4 : 0;
    const int64_t nln = H * 2 * d * 4;
    const Range rQ{Q, nq}, rK{K, nq}, rV{V, nq}, rdY{dY, nq};
    const Range rW0{W0, units > 0 ? (w0_per_batch ? units : H) * n_state : 0};
    const Range rEta{eta, units > 0 ? H * 4 : 0}, rdWo{dW_out, units * n_state};
    const Range rEt{pro.eta_tok, ntok}, rLq{pro.ln_q, pro.ln_q ? nln : 0}, rLk{pro.ln_k, pro.ln_k ? nln : 0};
    const Range rdQ{dQ, nq}, rdK{dK, nq}, rdV{dV, nq};
    const Range rdW0{dW0, (w0_per_batch ? units : H) * n_state}, rdEta{deta, H * 4};
    const Range rdEt{deta_tok, deta_tok ? ntok : 0}, rdLq{dln_q, dln_q ? nln : 0}, rdLk{dln_k, dln_k ? nln : 0};
    const Range outs[] = {rdQ, rdK, rdV, rdW0, rdEta, rdEt, rdLq, rdLk};
    const Range all[] = {rQ, rK, rV, rdY, rW0, rEta, rdWo, rEt, rLq, rLk,
                         rdQ, rdK, rdV, rdW0, rdEta, rdEt, rdLq, rdLk};
    for (const Range& o : outs) {
        int hits = 0;   // an output overlaps itself once
        for (const Range& x : all)
            hits += overlap(o, x) ? 1 : 0;
        if (hits > 1) return TTT_ERR_INVALID_ARG;
    }

    ttt::LinearBwdArgs a{Q, K, V, qkv_dtype, W0, w0_per_batch, eta, B, H, T, d, b,
                         dY, dW_out, dQ, dK, dV, dW0, deta, static_cast<hipStream_t>(stream)};
    a.pro = pro;
    a.deta_tok = deta_tok;
    a.dln_q = dln_q;
    a.dln_k = dln_k;
    if (!ttt::linear_backward_supports(a)) return TTT_ERR_UNSUPPORTED;
    ttt::SegmentPlan p;
    if (units > 0)
        p = plan_backward(units, T, b, qkv_dtype == TTT_BF16 ? ttt::kLinearBwdBf16Costs
                                                              : ttt::kLinearBwdF32Costs);
    void* ws = nullptr;
    if (workspace_get(&ws, ttt::linear_backward_workspace_bytes(a, p), a.stream) != hipSuccess)
        return TTT_ERR_HIP;
    return hip_status(ttt::launch_linear_backward(a, p, ws));
}

}  // namespace

extern "C" {

int ttt_linear_backward(const void* Q, const void* K, const void* V, int qkv_dtype,
                        const float* W0, int w0_per_batch, const float* eta,
                        int64_t B, int64_t H, int64_t T, int d, int b,
                        const void* dY, const float* dW_out,
                        void* dQ, void* dK, void* dV, float* dW0, float* deta, void* stream)
{
    return linear_backward_impl(Q, K, V, qkv_dtype, W0, w0_per_batch, eta, B, H, T, d, b, dY,
                                dW_out, dQ, dK, dV, dW0, deta, ttt::Prologue{}, nullptr, nullptr,
                                nullptr, stream);
}

int ttt_linear_backward_ex(const void* Q, const void* K, const void* V, int qkv_dtype,
                           const float* W0, int w0_per_batch, const float* eta,
                           const float* eta_tok, const float* ln_q, const float* ln_k,
                           float ln_eps, int read_mode, int64_t B, int64_t H, int64_t T, int d,
                           int b, const void* dY, const float* dW_out, void* dQ, void* dK,
                           void* dV, float* dW0, float* deta, float* deta_tok, float* dln_q,
                           float* dln_k, void* stream)
{
    if ((ln_q || ln_k) && !(ln_eps > 0.0f && ln_eps < 1e30f))
        return TTT_ERR_INVALID_ARG;
    if (read_mode != 0 && read_mode != 1)
        return TTT_ERR_INVALID_ARG;
    ttt::Prologue pro;
    pro.eta_tok = eta_tok;
    pro.ln_q = ln_q;
    pro.ln_k = ln_k;
    pro.ln_eps = ln_eps;
    pro.read_start = read_mode;
    return linear_backward_impl(Q, K, V, qkv_dtype, W0, w0_per_batch, eta, B, H, T, d, b, dY,
                                dW_out, dQ, dK, dV, dW0, deta, pro, deta_tok, dln_q, dln_k, stream);
}

int ttt_linear_backward_segments(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype)
{
    if (B < 0 || H < 0 || T < 0 || b < 1) return TTT_ERR_INVALID_ARG;
    if (!valid_dtype(qkv_dtype) || d != 64 || b != 16) return TTT_ERR_UNSUPPORTED;
    int64_t units = B;
    if (!mul_ok(units, H) || units > kMaxUnits) return TTT_ERR_UNSUPPORTED;
    if (units == 0 || T == 0) return 1;
    return plan_backward(units, T, b, qkv_dtype == TTT_BF16 ? ttt::kLinearBwdBf16Costs
                                                            : ttt::kLinearBwdF32Costs).nseg;
}

int ttt_mlp_forward(const void* Q, const void* K, const void* V, int qkv_dtype,
                    const float* W1_0, const float* W2_0, int w0_per_batch,
                    const float* eta, int64_t B, int64_t H, int64_t T, int d, int m, int b,
                    void* Y, float* W1_out, float* W2_out, void* stream)
{
    if (B < 0 || H < 0 || T < 0 || b < 1 || m < 1 || (w0_per_batch != 0 && w0_per_batch != 1))
        return TTT_ERR_INVALID_ARG;
    if (!valid_dtype(qkv_dtype) || !(d == 16 || d == 32 || d == 64) || b > 64 ||
        m % 16 != 0 || m > 512)
        return TTT_ERR_UNSUPPORTED;
    int64_t units = B;
    if (!mul_ok(units, H) || units > kMaxUnits) return TTT_ERR_UNSUPPORTED;
    if (units == 0) return TTT_OK;
    int64_t n_qkv = units;
    if (!mul_ok(n_qkv, T) || !mul_ok(n_qkv, d) || !mul_ok(n_qkv, 4)) return TTT_ERR_UNSUPPORTED;
    n_qkv = n_qkv / 4 * static_cast<int64_t>(elem_bytes(qkv_dtype));
    const int64_t n_state = static_cast<int64_t>(d) * m * 4;
    if (!W1_0 || !W2_0 || !eta || !W1_out || !W2_out) return TTT_ERR_INVALID_ARG;
    if (T > 0 && (!Q || !K || !V || !Y)) return TTT_ERR_INVALID_ARG;

    const int64_t n_src = (w0_per_batch ? units : H) * n_state;
    const Range rQ{Q, T ? n_qkv : 0}, rK{K, T ? n_qkv : 0}, rV{V, T ? n_qkv : 0};
    const Range rY{Y, T ? n_qkv : 0};
    const Range rW1{W1_0, n_src}, rW2{W2_0, n_src};
    const Range rW1o{W1_out, units * n_state}, rW2o{W2_out, units * n_state};
    const Range rEta{eta, H * 4};
    for (const Range& in : {rQ, rK, rV, rW1, rW2, rEta, rW1o, rW2o})
        if (overlap(rY, in)) return TTT_ERR_INVALID_ARG;
    for (const Range& in : {rQ, rK, rV, rEta, rW2, rW2o})
        if (overlap(rW1o, in)) return TTT_ERR_INVALID_ARG;
    for (const Range& in : {rQ, rK, rV, rEta, rW1})
        if (overlap(rW2o, in)) return TTT_ERR_INVALID_ARG;
    if (overlap(rW1o, rW1) && !(w0_per_batch && static_cast<const void*>(W1_out) == W1_0))
        return TTT_ERR_INVALID_ARG;
    if (overlap(rW2o, rW2) && !(w0_per_batch && static_cast<const void*>(W2_out) == W2_0))
        return TTT_ERR_INVALID_ARG;

    MlpArgs a{Q, K, V, qkv_dtype, W1_0, W2_0, w0_per_batch, eta, B, H, T, d, m, b,
              Y, W1_out, W2_out, static_cast<hipStream_t>(stream)};
    if (ttt::mlp_mfma_supports(a))
        return hip_status(ttt::launch_mlp_mfma(a));
    if (ttt::mlp_generic_lds_bytes(d, m, b) > static_cast<size_t>(ttt::kMaxLdsBytes))
        return TTT_ERR_UNSUPPORTED;
    return hip_status(ttt::launch_mlp_generic(a));
}

}  // extern "C"

namespace {

int decode_impl(const void* q, const void* k, const void* v, int qkv_dtype, float* W,
                const float* eta, int64_t B, int64_t H, int d, void* y, void* stream,
                const ttt::Prologue& pro)
{
    if (B < 0 || H < 0) return TTT_ERR_INVALID_ARG;
    if (!valid_dtype(qkv_dtype) || !d_supported(d)) return TTT_ERR_UNSUPPORTED;
    int64_t units = B;
    if (!mul_ok(units, H) || units > kMaxUnits) return TTT_ERR_UNSUPPORTED;
    if (units == 0) return TTT_OK;
    if (!q || !k || !v || !W || !eta || !y) return TTT_ERR_INVALID_ARG;
    const int64_t n_vec = units * d * static_cast<int64_t>(elem_bytes(qkv_dtype));
    const Range rq{q, n_vec}, rk{k, n_vec}, rv{v, n_vec}, ry{y, n_vec};
    const Range rW{W, units * d * d * 4}, rEta{eta, H * 4};
    for (const Range& in : {rq, rk, rv, rW, rEta})
        if (overlap(ry, in)) return TTT_ERR_INVALID_ARG;
    for (const Range& in : {rq, rk, rv, rEta})
        if (overlap(rW, in)) return TTT_ERR_INVALID_ARG;
    if (pro.active()) {
        const Range rTok{pro.eta_tok, pro.eta_tok ? units * 4 : 0};
        const Range rLq{pro.ln_q, pro.ln_q ? H * 2 * d * 4 : 0}, rLk{pro.ln_k, pro.ln_k ? H * 2 * d * 4 : 0};
        for (const Range& in : {rTok, rLq, rLk})
            if (overlap(ry, in) || overlap(rW, in)) return TTT_ERR_INVALID_ARG;
    }
    DecodeArgs a{q, k, v, qkv_dtype, W, eta, B, H, d, y, static_cast<hipStream_t>(stream)};
    a.pro = pro;
    return hip_status(ttt::launch_decode(a));
}

}  // namespace

extern "C" {

int ttt_linear_decode_step(const void* q, const void* k, const void* v, int qkv_dtype,
                           float* W, const float* eta, int64_t B, int64_t H, int d,
                           void* y, void* stream)
{
    return decode_impl(q, k, v, qkv_dtype, W, eta, B, H, d, y, stream, ttt::Prologue{});
}

int ttt_linear_decode_step_ex(const void* q, const void* k, const void* v, int qkv_dtype,
                              float* W, const float* eta, const float* eta_tok,
                              const float* ln_q, const float* ln_k, float ln_eps, int read_mode,
                              int64_t B, int64_t H, int d, void* y, void* stream)
{
    if ((ln_q || ln_k) && !(ln_eps > 0.0f && ln_eps < 1e30f))
        return TTT_ERR_INVALID_ARG;
    if (read_mode != 0 && read_mode != 1)
        return TTT_ERR_INVALID_ARG;
    ttt::Prologue pro;
    pro.eta_tok = eta_tok;
    pro.ln_q = ln_q;
    pro.ln_k = ln_k;
    pro.ln_eps = ln_eps;
    pro.read_start = read_mode;
    return decode_impl(q, k, v, qkv_dtype, W, eta, B, H, d, y, stream, pro);
}

}  // extern "C"
