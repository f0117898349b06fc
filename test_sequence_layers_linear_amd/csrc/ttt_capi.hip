// ttt_capi.hip -- the C ABI declared in include/ttt.h: argument validation,
// kernel selection and launch on the caller's stream.  Validation happens
// before any HIP call, so every error path is reachable without a GPU.
#include "ttt.h"
#include "ttt_internal.h"

#include <stdint.h>

#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <functional>
#include <mutex>

namespace {

using ttt::LinearArgs;
using ttt::MlpArgs;
using ttt::DecodeArgs;
using ttt::MomentumArgs;

constexpr int kAbiVersion = (2 << 16) | 3;

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

// most (batch, head) chains: a launch's grid, counted in work-items, must
// stay below 2^32 (the widest launch has up to 768 threads per chain)
constexpr int64_t kMaxUnits = int64_t{1} << 20;
// longest sequence: every kernel indexes a chain's tokens with 32-bit ints
// (the MFMA kernels' byte offsets are bounded tighter by their own checks)
constexpr int64_t kMaxTokens = 0x7fffffff;

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

// Workspace of a segmented forward with S segments per chain: the maps of
// segments 0..S-2 ([units][S-1][2][d][d]) and the start states
// ([units][S][d][d]), fp32.  One segment needs none.
int64_t forward_workspace_bytes(int64_t units, int d, int S)
{
    if (S <= 1) return 0;
    return units * (3 * static_cast<int64_t>(S) - 2) * d * d * static_cast<int64_t>(sizeof(float));
}

ttt::SegmentPlan with_segments(int64_t T, int chunk, int S)
{
    ttt::SegmentPlan p;
    p.seg_len = T;
    const int64_t chunks = (T + chunk - 1) / chunk;
    if (S > 1 && chunks > 0) {
        p.seg_len = ((chunks + S - 1) / S) * chunk;
        p.nseg = static_cast<int>((T + p.seg_len - 1) / p.seg_len);
    }
    return p;
}

// Segment count for a chain-parallel scan of `units` chains of T tokens in
// units of `chunk` tokens, whose maps and start states for S segments must
// fit the workspace (`fits`).  Each launch of the split runs all its
// workgroups at once, one per CU (more would queue or share CUs and stretch
// the slowest ones), so S is limited to what fits; within that it minimises
//   ceil(chunks / S) (map + fwd) + (S - 1) apply + launch
// against the unsplit chunks * fwd (costs measured on MI355X).
// The environment variable `env_name` = S (1 <= S <= max_s) forces S
// segments (at least one chunk each; fewer if the workspace is too small),
// for tests and tuning.
ttt::SegmentPlan plan_split(int64_t units, int64_t T, int chunk, const ttt::SegmentCosts& cost,
                            const std::function<bool(int)>& fits, const char* env_name, int max_s)
{
    const int64_t chunks = (T + chunk - 1) / chunk;
    if (const char* env = getenv(env_name)) {
        long S = std::min<long>(strtol(env, nullptr, 10), max_s);
        if (S >= 1 && chunks > 0) {
            S = std::min<long>(S, chunks);
            while (S > 1 && !fits(static_cast<int>(with_segments(T, chunk, static_cast<int>(S)).nseg)))
                --S;
            return with_segments(T, chunk, static_cast<int>(S));
        }
    }
    const int64_t cus = device_cus();
    const int64_t scan_blocks = units * cost.scan_blocks_per_segment;
    if (cus <= 0 || 2 * scan_blocks > cus || chunks < 4) return with_segments(T, chunk, 1);
    double best = static_cast<double>(chunks) * cost.fwd;
    int best_s = 1;
    for (int S = 2; S <= max_s; ++S) {
        if (scan_blocks * S > cus ||
            units * (S - 1) * cost.map_blocks_per_segment > cost.map_blocks_per_cu * cus)
            break;
        const int64_t per = (chunks + S - 1) / S;
        if (per < 2) break;
        if (!fits(with_segments(T, chunk, S).nseg)) continue;
        const double t = per * (cost.map + cost.fwd) + (S - 1) * cost.apply + cost.launch;
        if (t < best) { best = t; best_s = S; }
    }
    return with_segments(T, chunk, best_s);
}

ttt::SegmentPlan plan_segments(int64_t units, int64_t T, int chunk, int d,
                               const ttt::SegmentCosts& cost, int64_t ws_bytes)
{
    return plan_split(units, T, chunk, cost,
                      [&](int S) { return forward_workspace_bytes(units, d, S) <= ws_bytes; },
                      "TTT_LINEAR_SEGMENTS", ttt::kMaxSegments);
}

// Segment count for the backward of a TTT-Linear scan: each segment pays
// its chunks' forward map, cotangent map and backward, and the two
// compositions (S - 1) steps each, plus four extra launches.  Up to
// max_per_cu segment-backward workgroups share a CU, each slowed by `share`
// per extra workgroup per CU; the maps launches may hold maps_per_cu per CU.
// TTT_LINEAR_BWD_SEGMENTS=S forces S segments.
ttt::SegmentPlan plan_backward(int64_t units, int64_t T, int chunk, const ttt::BwdCosts& cost,
                               const std::function<bool(const ttt::SegmentPlan&)>& fits)
{
    const int64_t chunks = (T + chunk - 1) / chunk;
    if (const char* env = getenv("TTT_LINEAR_BWD_SEGMENTS")) {
        long S = std::min<long>(strtol(env, nullptr, 10), ttt::kMaxSegments);
        if (S >= 1 && chunks > 0) {
            S = std::min<long>(S, chunks);
            while (S > 1 && !fits(with_segments(T, chunk, static_cast<int>(S))))
                --S;
            return with_segments(T, chunk, static_cast<int>(S));
        }
    }
    ttt::SegmentPlan p = with_segments(T, chunk, 1);
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
        if (t < best && fits(with_segments(T, chunk, S))) { best = t; best_s = S; }
    }
    return with_segments(T, chunk, best_s);
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

// Runs a (possibly segmented) MFMA linear scan with the maps and start
// states in the caller's workspace (planned to fit it).  The start states
// (including the copy of W0 for the first segment) are complete before any
// segment writes W_out, so W_out may overwrite W0.
int run_linear_segmented(LinearArgs a, ttt::SegmentPlan p, void* ws,
                         hipError_t (*launch)(const LinearArgs&, const ttt::SegmentPlan&))
{
    if (p.nseg <= 1) return hip_status(launch(a, p));
    const int64_t units = a.B * a.H;
    const size_t state = static_cast<size_t>(a.d) * a.d * sizeof(float);
    const size_t map_bytes = static_cast<size_t>(units) * (p.nseg - 1) * 2 * state;
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

// The MFMA scan (with its segment costs) that runs a TTT-Linear forward, or
// none (the generic kernel: never segmented).
struct LinearScan {
    const ttt::SegmentCosts* cost;
    hipError_t (*launch)(const LinearArgs&, const ttt::SegmentPlan&);
};

LinearScan pick_scan(const LinearArgs& a)
{
    if (ttt::linear_mfma_supports(a)) return {&ttt::kLinearBf16Costs, ttt::launch_linear_mfma};
    if (use_cols_f32(a)) return {&ttt::kLinearF32ColsCosts, ttt::launch_linear_cols_f32};
    if (ttt::linear_mfma_f32_supports(a)) return {&ttt::kLinearF32Costs, ttt::launch_linear_mfma_f32};
    return {nullptr, nullptr};
}

// The fused layout with S segments (bf16 TTT-Linear, with or without the
// prologue):
// segment 0 of L0 chunks, scanned beside the maps of segments 1 .. S - 2 of L
// chunks each, L0 = ratio L so that the two roles of the first launch end
// together; the last segment takes the rest.  nseg = 1 if S does not fit.
ttt::SegmentPlan fused_with_segments(int64_t T, int chunk, int S, double ratio)
{
    ttt::SegmentPlan p = with_segments(T, chunk, 1);
    const int64_t chunks = (T + chunk - 1) / chunk;
    if (S < 3) return p;
    const int64_t L = static_cast<int64_t>(std::ceil(chunks / (S - 1 + ratio)));
    const int64_t L0 = std::max<int64_t>(1, chunks - (S - 1) * L);
    if (L0 + (S - 2) * L >= chunks) return p;       // the last segment would be empty
    p.nseg = S;
    p.seg_len = L * chunk;
    p.first_len = L0 * chunk;
    p.fused = true;
    return p;
}

// Estimated duration (us) of a bf16 TTT-Linear plan, from the segment costs:
// unfused, the longest segment's map and scan; fused, the longer role of the
// first launch, then a segment's scan.
double plan_cost(const ttt::SegmentPlan& p, int64_t T, int chunk, const ttt::SegmentCosts& cost)
{
    const int64_t chunks = (T + chunk - 1) / chunk;
    if (p.nseg <= 1) return static_cast<double>(chunks) * cost.fwd;
    const double L = static_cast<double>(p.seg_len / chunk);
    if (!p.fused) return L * (cost.map + cost.fwd) + (p.nseg - 1) * cost.apply + cost.launch;
    const double L0 = static_cast<double>(p.first() / chunk);
    return std::max(L0 * cost.fwd * ttt::kStagedScanFactor, L * cost.map) +
           (p.nseg - 2) * cost.apply + cost.launch + L * cost.fwd;
}

// The plan a forward of these sizes uses with `ws_bytes` of workspace.  The
// bf16 MFMA scan also weighs the fused layout (off with
// TTT_LINEAR_FUSED=0): its two launches hold units (S - 1) workgroups each,
// so it may use one more segment than the unfused layout on the same CUs.
ttt::SegmentPlan plan_forward(const LinearArgs& a, int64_t ws_bytes)
{
    const LinearScan k = pick_scan(a);
    const int64_t units = a.B * a.H;
    if (!k.cost || units == 0 || a.T == 0) return with_segments(a.T, a.b, 1);
    const ttt::SegmentPlan unfused = plan_segments(units, a.T, a.b, a.d, *k.cost, ws_bytes);
    const char* off = getenv("TTT_LINEAR_FUSED");
    if (k.cost != &ttt::kLinearBf16Costs || (off && strtol(off, nullptr, 10) == 0))
        return unfused;
    const ttt::SegmentCosts& cost = *k.cost;
    const double ratio = cost.map / (cost.fwd * ttt::kStagedScanFactor);
    auto fits = [&](const ttt::SegmentPlan& p) {
        return forward_workspace_bytes(units, a.d, p.nseg) <= ws_bytes;
    };
    if (getenv("TTT_LINEAR_SEGMENTS")) {         // forced: the same count, fused when it can be
        const ttt::SegmentPlan f = fused_with_segments(a.T, a.b, unfused.nseg, ratio);
        return f.fused && f.nseg == unfused.nseg && fits(f) ? f : unfused;
    }
    const int64_t cus = device_cus();
    ttt::SegmentPlan best = unfused;
    double best_t = plan_cost(unfused, a.T, a.b, cost);
    for (int S = 3; S <= ttt::kMaxSegments && cus > 0 && units * (S - 1) <= cus; ++S) {
        const ttt::SegmentPlan f = fused_with_segments(a.T, a.b, S, ratio);
        if (!f.fused || !fits(f)) continue;
        const double t = plan_cost(f, a.T, a.b, cost);
        if (t < best_t) { best = f; best_t = t; }
    }
    return best;
}

// Size checks shared by the TTT-Linear entry points and their queries.
int linear_sizes_status(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype)
{
    if (B < 0 || H < 0 || T < 0 || b < 1) return TTT_ERR_INVALID_ARG;
    if (!valid_dtype(qkv_dtype) || !d_supported(d) || b > 64) return TTT_ERR_UNSUPPORTED;
    int64_t units = B;
    if (!mul_ok(units, H) || units > kMaxUnits || T > kMaxTokens) return TTT_ERR_UNSUPPORTED;
    int64_t n = units;
    if (!mul_ok(n, T) || !mul_ok(n, d) || !mul_ok(n, 4)) return TTT_ERR_UNSUPPORTED;
    return TTT_OK;
}

// Scratch of ttt_linear_forward_noalloc: the segment maps and start states
// of one call, in a file-scope device array instead of caller memory.  Every
// device the library runs on holds its own copy until the process ends.
constexpr int64_t kScratchBytes = int64_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on the device that `stream` belongs to (the
// null stream: the current device), looked up once per device with that
// device current (the array's name is not a device address in host code,
// and each device holds its own copy at its own address).
int scratch_address(hipStream_t stream, void** out)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices];
    int cur = 0, dev = 0;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &dev) != hipSuccess ||
        dev < 0 || dev >= kMaxDevices)
        return TTT_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return TTT_ERR_HIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return TTT_ERR_HIP;
        if (e != hipSuccess || !p) return TTT_ERR_HIP;
        addr[dev] = p;
    }
    *out = addr[dev];
    return TTT_OK;
}

// ttt_linear_forward with an optional input prologue (pro.active(): d = 64,
// b = 16 only) and the caller's workspace, or (use_scratch) the static
// scratch with the plan a sufficient workspace would get.
int linear_forward_impl(const void* Q, const void* K, const void* V, int qkv_dtype,
                        const float* W0, int w0_per_batch, const float* eta,
                        int64_t B, int64_t H, int64_t T, int d, int b,
                        void* Y, float* W_out, void* ws, int64_t ws_bytes, void* stream,
                        const ttt::Prologue& pro, bool use_scratch = false)
{
    if (w0_per_batch != 0 && w0_per_batch != 1) return TTT_ERR_INVALID_ARG;
    if (ws_bytes < 0 || (ws_bytes > 0 && !ws)) return TTT_ERR_INVALID_ARG;
    if (const int st = linear_sizes_status(B, H, T, d, b, qkv_dtype)) return st;
    const int64_t units = B * H;
    if (units == 0) return TTT_OK;
    const int64_t n_qkv = units * T * d * static_cast<int64_t>(elem_bytes(qkv_dtype));
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
    const Range rTok{pro.eta_tok, pro.eta_tok ? units * T * 4 : 0};
    const Range rLq{pro.ln_q, pro.ln_q ? H * 2 * d * 4 : 0}, rLk{pro.ln_k, pro.ln_k ? H * 2 * d * 4 : 0};
    for (const Range& in : {rTok, rLq, rLk})
        if (overlap(rY, in) || overlap(rWo, in)) return TTT_ERR_INVALID_ARG;
    const Range rWs{ws, ws_bytes};
    for (const Range& x : {rQ, rK, rV, rY, rW0, rWo, rEta, rTok, rLq, rLk})
        if (overlap(rWs, x)) return TTT_ERR_INVALID_ARG;

    LinearArgs a{Q, K, V, qkv_dtype, W0, w0_per_batch, eta, B, H, T, d, b,
                 Y, W_out, static_cast<hipStream_t>(stream)};
    a.pro = pro;
    if (pro.active() && !ttt::linear_mfma_supports(a) && !ttt::linear_mfma_f32_supports(a))
        return TTT_ERR_UNSUPPORTED;
    const LinearScan k = pick_scan(a);
    if (k.launch) {
        if (!use_scratch) return run_linear_segmented(a, plan_forward(a, ws_bytes), ws, k.launch);
        const ttt::SegmentPlan p = plan_forward(a, INT64_MAX);
        if (forward_workspace_bytes(units, d, p.nseg) > kScratchBytes) return TTT_ERR_UNSUPPORTED;
        void* sp = nullptr;
        if (p.nseg > 1)
            if (const int st = scratch_address(a.stream, &sp)) return st;
        return run_linear_segmented(a, p, sp, k.launch);
    }
    if (ttt::linear_generic_lds_bytes(d, b) > static_cast<size_t>(ttt::kMaxLdsBytes))
        return TTT_ERR_UNSUPPORTED;
    return hip_status(ttt::launch_linear_generic(a));
}


}  // namespace

extern "C" {

int ttt_linear_forward(const void* Q, const void* K, const void* V, int qkv_dtype,
                       const float* W0, int w0_per_batch, const float* eta,
                       int64_t B, int64_t H, int64_t T, int d, int b,
                       void* Y, float* W_out, void* workspace, int64_t workspace_bytes,
                       void* stream)
{
    return linear_forward_impl(Q, K, V, qkv_dtype, W0, w0_per_batch, eta, B, H, T, d, b, Y, W_out,
                               workspace, workspace_bytes, stream, ttt::Prologue{});
}

int ttt_linear_forward_ex(const void* Q, const void* K, const void* V, int qkv_dtype,
                          const float* W0, int w0_per_batch, const float* eta,
                          const float* eta_tok, const float* ln_q, const float* ln_k, float ln_eps,
                          int read_mode, int64_t B, int64_t H, int64_t T, int d, int b,
                          void* Y, float* W_out, void* workspace, int64_t workspace_bytes,
                          void* stream)
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
                               workspace, workspace_bytes, stream, pro);
}

int ttt_linear_forward_noalloc(const void* Q, const void* K, const void* V, int qkv_dtype,
                               const float* W0, int w0_per_batch, const float* eta,
                               int64_t B, int64_t H, int64_t T, int d, int b,
                               void* Y, float* W_out, void* stream)
{
    return linear_forward_impl(Q, K, V, qkv_dtype, W0, w0_per_batch, eta, B, H, T, d, b, Y, W_out,
                               nullptr, 0, stream, ttt::Prologue{}, true);
}

int64_t ttt_linear_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

int64_t ttt_linear_workspace_bytes(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype)
{
    if (const int st = linear_sizes_status(B, H, T, d, b, qkv_dtype)) return st;
    LinearArgs a{nullptr, nullptr, nullptr, qkv_dtype, nullptr, 0, nullptr, B, H, T, d, b,
                 nullptr, nullptr, nullptr};
    return forward_workspace_bytes(B * H, d, plan_forward(a, INT64_MAX).nseg);
}

int ttt_linear_segments(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype)
{
    if (const int st = linear_sizes_status(B, H, T, d, b, qkv_dtype)) return st;
    LinearArgs a{nullptr, nullptr, nullptr, qkv_dtype, nullptr, 0, nullptr, B, H, T, d, b,
                 nullptr, nullptr, nullptr};
    return plan_forward(a, INT64_MAX).nseg;
}

int ttt_linear_fused(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype)
{
    if (const int st = linear_sizes_status(B, H, T, d, b, qkv_dtype)) return st;
    LinearArgs a{nullptr, nullptr, nullptr, qkv_dtype, nullptr, 0, nullptr, B, H, T, d, b,
                 nullptr, nullptr, nullptr};
    return plan_forward(a, INT64_MAX).fused ? 1 : 0;
}

}  // extern "C"

namespace {

// Planner costs of a backward call: by input dtype, and for bf16 with or
// without the prologue.
const ttt::BwdCosts& bwd_costs(int qkv_dtype, bool pro)
{
    if (qkv_dtype != TTT_BF16) return ttt::kLinearBwdF32Costs;
    return pro ? ttt::kLinearBwdBf16ProCosts : ttt::kLinearBwdBf16Costs;
}

int linear_backward_impl(const void* Q, const void* K, const void* V, int qkv_dtype,
                         const float* W0, int w0_per_batch, const float* eta,
                         int64_t B, int64_t H, int64_t T, int d, int b,
                         const void* dY, const float* dW_out,
                         void* dQ, void* dK, void* dV, float* dW0, float* deta,
                         const ttt::Prologue& pro, float* deta_tok, float* dln_q, float* dln_k,
                         void* ws, int64_t ws_bytes, void* stream)
{
    if (w0_per_batch != 0 && w0_per_batch != 1) return TTT_ERR_INVALID_ARG;
    if (ws_bytes < 0 || (ws_bytes > 0 && !ws)) return TTT_ERR_INVALID_ARG;
    if (const int st = linear_sizes_status(B, H, T, d, b, qkv_dtype)) return st;
    if (d != 64 || b != 16) return TTT_ERR_UNSUPPORTED;
    const int64_t units = B * H;
    const int64_t n_qkv = units * T * d * static_cast<int64_t>(elem_bytes(qkv_dtype));
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
    const Range rWs{ws, ws_bytes};
    const Range outs[] = {rdQ, rdK, rdV, rdW0, rdEta, rdEt, rdLq, rdLk, rWs};
    const Range all[] = {rQ, rK, rV, rdY, rW0, rEta, rdWo, rEt, rLq, rLk,
                         rdQ, rdK, rdV, rdW0, rdEta, rdEt, rdLq, rdLk, rWs};
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
    auto fits = [&](const ttt::SegmentPlan& p) {
        return static_cast<int64_t>(ttt::linear_backward_workspace_bytes(a, p)) <= ws_bytes;
    };
    ttt::SegmentPlan p;
    if (units > 0)
        p = plan_backward(units, T, b, bwd_costs(qkv_dtype, pro.active()), fits);
    if (!fits(p)) return TTT_ERR_INVALID_ARG;   // not even one segment's states fit
    return hip_status(ttt::launch_linear_backward(a, p, ws));
}

// Backward arguments for a workspace query: shared W0 and the prologue's
// buffers, the most any variant of the call needs.
ttt::LinearBwdArgs bwd_query_args(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype)
{
    ttt::LinearBwdArgs a{nullptr, nullptr, nullptr, qkv_dtype, nullptr, 0, nullptr, B, H, T, d, b,
                         nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    a.pro.read_start = 1;
    return a;
}

}  // namespace

extern "C" {

int ttt_linear_backward(const void* Q, const void* K, const void* V, int qkv_dtype,
                        const float* W0, int w0_per_batch, const float* eta,
                        int64_t B, int64_t H, int64_t T, int d, int b,
                        const void* dY, const float* dW_out,
                        void* dQ, void* dK, void* dV, float* dW0, float* deta,
                        void* workspace, int64_t workspace_bytes, void* stream)
{
    return linear_backward_impl(Q, K, V, qkv_dtype, W0, w0_per_batch, eta, B, H, T, d, b, dY,
                                dW_out, dQ, dK, dV, dW0, deta, ttt::Prologue{}, nullptr, nullptr,
                                nullptr, workspace, workspace_bytes, stream);
}

int ttt_linear_backward_ex(const void* Q, const void* K, const void* V, int qkv_dtype,
                           const float* W0, int w0_per_batch, const float* eta,
                           const float* eta_tok, const float* ln_q, const float* ln_k,
                           float ln_eps, int read_mode, int64_t B, int64_t H, int64_t T, int d,
                           int b, const void* dY, const float* dW_out, void* dQ, void* dK,
                           void* dV, float* dW0, float* deta, float* deta_tok, float* dln_q,
                           float* dln_k, void* workspace, int64_t workspace_bytes, void* stream)
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
                                dW_out, dQ, dK, dV, dW0, deta, pro, deta_tok, dln_q, dln_k,
                                workspace, workspace_bytes, stream);
}

int ttt_linear_backward_segments(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype)
{
    if (const int st = linear_sizes_status(B, H, T, d, b, qkv_dtype)) return st;
    if (d != 64 || b != 16) return TTT_ERR_UNSUPPORTED;
    if (B * H == 0 || T == 0) return 1;
    return plan_backward(B * H, T, b, bwd_costs(qkv_dtype, false),
                         [](const ttt::SegmentPlan&) { return true; }).nseg;
}

int64_t ttt_linear_backward_workspace_bytes(int64_t B, int64_t H, int64_t T, int d, int b,
                                            int qkv_dtype)
{
    if (const int st = linear_sizes_status(B, H, T, d, b, qkv_dtype)) return st;
    if (d != 64 || b != 16) return TTT_ERR_UNSUPPORTED;
    const ttt::LinearBwdArgs a = bwd_query_args(B, H, T, d, b, qkv_dtype);
    // enough for the plain call's plan and the prologue call's, which may
    // take more segments
    size_t bytes = ttt::linear_backward_workspace_bytes(a, ttt::SegmentPlan{});
    if (B * H > 0 && T > 0) {
        for (const bool pro : {false, true}) {
            const ttt::SegmentPlan p = plan_backward(B * H, T, b, bwd_costs(qkv_dtype, pro),
                                                     [](const ttt::SegmentPlan&) { return true; });
            bytes = std::max(bytes, ttt::linear_backward_workspace_bytes(a, p));
        }
    }
    return static_cast<int64_t>(bytes);
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
    if (!mul_ok(units, H) || units > kMaxUnits || T > kMaxTokens) return TTT_ERR_UNSUPPORTED;
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
    // the step reads rows of q, k and W with 16-byte loads
    for (const void* ptr : {q, k, static_cast<const void*>(W)})
        if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return TTT_ERR_INVALID_ARG;
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

namespace {

// Tokens per unit of a momentum segment: a stage of two chunks (the chunk
// inverses are stored per stage).
constexpr int kMomentumStage = 32;

// Segments of a momentum forward of these sizes with `ws_bytes` of
// workspace (the bf16 MFMA scan only; one segment otherwise).
// TTT_MOMENTUM_SEGMENTS=S forces S segments.
ttt::SegmentPlan plan_momentum(const MomentumArgs& a, int64_t ws_bytes)
{
    const int64_t units = a.B * a.H;
    if (!ttt::momentum_mfma_supports(a) || units == 0 || a.T == 0)
        return with_segments(a.T, kMomentumStage, 1);
    const ttt::SegmentCosts& cost =
        a.grad_mode == 0 ? ttt::kMomentumExactCosts : ttt::kMomentumChunkStartCosts;
    return plan_split(units, a.T, kMomentumStage, cost,
                      [&](int S) {
                          return S <= 1 || (S <= ttt::kMaxMomentumSegments &&
                                            ttt::momentum_combine_lds_bytes(S) <=
                                                static_cast<size_t>(ttt::kMaxLdsBytes) &&
                                            ttt::momentum_mfma_workspace_bytes(a, S) <= ws_bytes);
                      },
                      "TTT_MOMENTUM_SEGMENTS", ttt::kMaxMomentumSegments);
}

// The launch configuration a momentum forward of these sizes takes: the
// workspace bytes it needs with `ws_bytes` available (INT64_MAX: the planned
// split's; the least is that of one segment), or a negative ttt_status.
int64_t momentum_plan(const MomentumArgs& a, int64_t ws_bytes = INT64_MAX)
{
    if (const int st = linear_sizes_status(a.B, a.H, a.T, a.d, a.b, a.dtype)) return st;
    if (a.grad_mode != 0 && a.grad_mode != 1) return TTT_ERR_INVALID_ARG;
    if (ttt::momentum_mfma_supports(a))
        return ttt::momentum_mfma_workspace_bytes(a, plan_momentum(a, ws_bytes).nseg);
    if (ttt::momentum_generic_lds_bytes(a.d, a.b) > static_cast<size_t>(ttt::kMaxLdsBytes))
        return TTT_ERR_UNSUPPORTED;
    return 0;
}

}  // namespace

extern "C" {

int ttt_linear_momentum_forward(const void* Q, const void* K, const void* V, int qkv_dtype,
                                const float* W0, int w0_per_batch, const float* M0,
                                const float* eta, const float* beta, int grad_mode,
                                int64_t B, int64_t H, int64_t T, int d, int b,
                                void* Y, float* W_out, float* M_out,
                                void* workspace, int64_t workspace_bytes, void* stream)
{
    if (w0_per_batch != 0 && w0_per_batch != 1) return TTT_ERR_INVALID_ARG;
    if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace)) return TTT_ERR_INVALID_ARG;
    MomentumArgs a{Q, K, V, qkv_dtype, W0, w0_per_batch, M0, eta, beta, grad_mode,
                   B, H, T, d, b, Y, W_out, M_out, static_cast<hipStream_t>(stream)};
    // the least workspace: that of one segment
    const int64_t need = momentum_plan(a, 0);
    if (need < 0) return static_cast<int>(need);
    const int64_t units = B * H;
    if (units == 0) return TTT_OK;
    if (!W0 || !eta || !beta || !W_out || !M_out) return TTT_ERR_INVALID_ARG;
    if (T > 0 && (!Q || !K || !V || !Y)) return TTT_ERR_INVALID_ARG;
    if (workspace_bytes < need) return TTT_ERR_INVALID_ARG;

    const int64_t n_qkv = units * T * d * static_cast<int64_t>(elem_bytes(qkv_dtype));
    const int64_t n_state = static_cast<int64_t>(d) * d * 4;
    const Range rQ{Q, T ? n_qkv : 0}, rK{K, T ? n_qkv : 0}, rV{V, T ? n_qkv : 0};
    const Range rY{Y, T ? n_qkv : 0};
    const Range rW0{W0, (w0_per_batch ? units : H) * n_state}, rM0{M0, M0 ? units * n_state : 0};
    const Range rWo{W_out, units * n_state}, rMo{M_out, units * n_state};
    const Range rEta{eta, H * 4}, rBeta{beta, H * 4}, rWs{workspace, workspace_bytes};
    for (const Range& in : {rQ, rK, rV, rW0, rM0, rEta, rBeta, rWo, rMo, rWs})
        if (overlap(rY, in)) return TTT_ERR_INVALID_ARG;
    for (const Range& in : {rQ, rK, rV, rEta, rBeta, rMo, rWs})
        if (overlap(rWo, in)) return TTT_ERR_INVALID_ARG;
    for (const Range& in : {rQ, rK, rV, rEta, rBeta, rW0, rWs})
        if (overlap(rMo, in)) return TTT_ERR_INVALID_ARG;
    if (overlap(rWo, rW0) && !(w0_per_batch && static_cast<const void*>(W_out) == W0))
        return TTT_ERR_INVALID_ARG;
    if (overlap(rWo, rM0) || (overlap(rMo, rM0) && M_out != M0)) return TTT_ERR_INVALID_ARG;
    for (const Range& in : {rQ, rK, rV, rW0, rM0, rEta, rBeta})
        if (overlap(rWs, in)) return TTT_ERR_INVALID_ARG;

    if (ttt::momentum_mfma_supports(a)) {
        const ttt::SegmentPlan p = plan_momentum(a, workspace_bytes);
        return hip_status(ttt::launch_momentum_mfma(a, workspace, p.nseg, p.seg_len));
    }
    return hip_status(ttt::launch_momentum_generic(a));
}

int64_t ttt_linear_momentum_workspace_bytes(int64_t B, int64_t H, int64_t T, int d, int b,
                                            int qkv_dtype, int grad_mode)
{
    MomentumArgs a{};
    a.dtype = qkv_dtype;
    a.grad_mode = grad_mode;
    a.B = B; a.H = H; a.T = T; a.d = d; a.b = b;
    return momentum_plan(a);
}

int ttt_linear_momentum_segments(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype,
                                 int grad_mode)
{
    MomentumArgs a{};
    a.dtype = qkv_dtype;
    a.grad_mode = grad_mode;
    a.B = B; a.H = H; a.T = T; a.d = d; a.b = b;
    const int64_t st = momentum_plan(a);
    if (st < 0) return static_cast<int>(st);
    return plan_momentum(a, INT64_MAX).nseg;
}

}  // extern "C"
