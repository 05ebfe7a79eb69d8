// moe_api.hip -- the C ABI of libmoe.so (declared in include/moe.h).
//
// Host side only: argument validation (before any launch), workspace
// carve-up, and the launch sequence of each entry point on the caller's
// stream.  No device memory is allocated here and no host synchronisation
// happens on the hot path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "moe.h"
#include "moe_kernels.h"

namespace moe {

static thread_local std::string g_err;
static thread_local std::vector<hipEvent_t> g_events;
static thread_local bool g_events_armed = false;

static int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int device_cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

struct Geo {
    int64_t T, d, E, k, dff, cap, max_rows;
    int esz;      // bytes per element of x / W / h
    int BT, nblk; // dispatch token blocks
    bool mfma_gate; // gate on matrix cores (bf16 x, E <= 256)
    bool rank_route; // k above the register groups' 32: logits, then the selection by rank
};

// cap = min(T, ceil(cf * T * k / E)); cf <= 0: no limit.  cf*T*k is exact in
// double for T*k < 2^29; the ceiling is settled with integer-valued products.
static int64_t capacity_of(int64_t T, int64_t E, int64_t k, float cf) {
    if (!(cf > 0.0f)) return T;
    const double q = (double)cf * (double)T * (double)k;
    int64_t c = (int64_t)std::ceil(q / (double)E);
    while (c > 1 && (double)(c - 1) * (double)E >= q) --c;
    while ((double)c * (double)E < q) ++c;
    return c < T ? c : T;
}

static int validate(const moe_shape* s, Geo* g) {
    if (s == nullptr) return fail(MOE_ERR_NULL, "shape is NULL");
    if (s->T < 1) return fail(MOE_ERR_SHAPE, "T must be >= 1 (got %lld)", (long long)s->T);
    if (s->E < 1 || s->E > 1024) return fail(MOE_ERR_SHAPE, "E must be in [1, 1024] (got %lld)", (long long)s->E);
    if (s->k < 1 || s->k > s->E)
        return fail(MOE_ERR_SHAPE, "k must be in [1, E] (got k=%lld, E=%lld)", (long long)s->k, (long long)s->E);
    if (s->d < 8 || s->d % 8 != 0) return fail(MOE_ERR_SHAPE, "d must be a positive multiple of 8 (got %lld)", (long long)s->d);
    if (s->d_ff < 8 || s->d_ff % 8 != 0)
        return fail(MOE_ERR_SHAPE, "d_ff must be a positive multiple of 8 (got %lld)", (long long)s->d_ff);
    if (!(s->temperature > 0.0f) || !std::isfinite(s->temperature))
        return fail(MOE_ERR_SHAPE, "temperature must be finite and > 0");
    if (!std::isfinite(s->capacity_factor)) return fail(MOE_ERR_SHAPE, "capacity_factor must be finite");
    if (!std::isfinite(s->aux_lambda)) return fail(MOE_ERR_SHAPE, "aux_lambda must be finite");
    if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return fail(MOE_ERR_SHAPE, "dtype must be MOE_F32 or MOE_BF16");
    if (s->T * s->k >= (int64_t(1) << 31)) return fail(MOE_ERR_SHAPE, "T*k must be < 2^31");
    if (s->d > (1 << 20) || s->d_ff > (1 << 20)) return fail(MOE_ERR_SHAPE, "d and d_ff must be <= 2^20");
    // one expert matrix must stay below 2^30 elements (32-bit byte offsets in the GEMMs)
    if (s->d * s->d_ff > (int64_t(1) << 29)) return fail(MOE_ERR_SHAPE, "d * d_ff must be <= 2^29");
    if (g) {
        g->T = s->T;
        g->d = s->d;
        g->E = s->E;
        g->k = s->k;
        g->dff = s->d_ff;
        g->cap = capacity_of(s->T, s->E, s->k, s->capacity_factor);
        g->max_rows = std::min(s->T * s->k, s->E * g->cap);
        g->esz = s->dtype == MOE_BF16 ? 2 : 4;
        g->BT = dispatch_block_tokens(s->T, (int)s->E, (int)s->k);
        g->nblk = (int)((s->T + g->BT - 1) / g->BT);
        g->rank_route = s->k > kRouteGroupMaxK;
        // the selection by rank reads logits: the gate runs with no winners
        g->mfma_gate = route_mfma_supported(s->dtype, (int)s->E, g->rank_route ? 0 : (int)s->k);
    }
    return MOE_OK;
}

struct WsLayout {
    size_t gate, logits, blkhist, offsets, idx, w, perm, slot, xperm, xpt, h, out, total;
};

static size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

static WsLayout ws_layout(const Geo& g) {
    WsLayout L{};
    size_t p = 0;
    auto take = [&](size_t bytes) {
        const size_t at = p;
        p = align_up(p + (bytes ? bytes : 1));
        return at;
    };
    L.gate = take(g.mfma_gate ? route_mfma_ws_bytes((int)g.d, (int)g.E) : 0);
    // k > 32: the logits the selection by rank reads, when the caller keeps none
    L.logits = take(g.rank_route ? sizeof(float) * (size_t)(g.T * g.E) : 0);
    L.blkhist = take(sizeof(int32_t) * (size_t)g.nblk * g.E);
    L.offsets = take(sizeof(int32_t) * (size_t)(g.E + 1));
    L.idx = take(sizeof(int32_t) * (size_t)(g.T * g.k));
    L.w = take(sizeof(float) * (size_t)(g.T * g.k));
    L.perm = take(sizeof(int32_t) * (size_t)g.max_rows);
    L.slot = take(sizeof(int32_t) * (size_t)(g.T * g.k));
    // row-major x_perm: fp32 layers only (a bf16 forward writes the tile copy below)
    L.xperm = take(g.esz == 4 ? (size_t)g.esz * (size_t)g.max_rows * g.d : 0);
    // bf16: x_perm again in the h tile layout, GEMM1's operand in moe_layer_forward
    L.xpt = take(g.esz == 2 ? (size_t)g.esz * (size_t)h_tiled_rows(g.max_rows, g.E) * (size_t)((g.d + 31) / 32 * 32)
                            : 0);
    // bf16: h in 16 x 32 tiles over 16-row-padded expert segments (ffn_bf16.hip)
    L.h = take(g.esz == 2 ? (size_t)g.esz * (size_t)h_tiled_rows(g.max_rows, g.E) * (size_t)((g.dff + 31) / 32 * 32)
                          : (size_t)g.esz * (size_t)g.max_rows * g.dff);
    L.out = take(sizeof(float) * (size_t)g.max_rows * g.d);
    L.total = p;
    return L;
}

static bool misaligned(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

#define MOE_REQUIRE(ptr)                                                        \
    do {                                                                        \
        if ((ptr) == nullptr) return fail(MOE_ERR_NULL, "%s is NULL", #ptr);   \
        if (misaligned(ptr)) return fail(MOE_ERR_ALIGN, "%s is not 16-byte aligned", #ptr); \
    } while (0)
#define MOE_OPTIONAL(ptr)                                                       \
    do {                                                                        \
        if (misaligned(ptr)) return fail(MOE_ERR_ALIGN, "%s is not 16-byte aligned", #ptr); \
    } while (0)
#define MOE_HIP(call, what)                                                     \
    do {                                                                        \
        hipError_t e_ = (call);                                                 \
        if (e_ != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e_)); \
    } while (0)

static int check_ws(const Geo& g, void* ws, size_t ws_bytes, WsLayout* L) {
    *L = ws_layout(g);
    if (ws == nullptr) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
    if (misaligned(ws)) return fail(MOE_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (ws_bytes < L->total)
        return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L->total);
    return MOE_OK;
}

template <typename T>
static T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// ---- static scratch of moe_dispatch_noalloc --------------------------------
// The dispatch's per-block expert histogram [nblk][E] int32 for callers that
// cannot allocate: a file-scope device array that every GPU the library runs
// on holds until the process ends.  In host code `scratch` names a host-side
// stand-in, not a device address: its address on each device comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that pointer is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_dev[64];   // device address of `scratch`, per device

static int scratch_on_current_device(void** out) {
    int dev = 0;
    MOE_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device %d: the scratch table holds 64 devices", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void* p = nullptr;
        MOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (p == nullptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return MOE_OK;
}

static const char* kStageNames[] = {"route", "hist", "scatter", "gather", "ffn1", "ffn2", "combine"};
constexpr int kNumStages = 7;

static void stage_event(int stage, int after, hipStream_t st) {
    if (!g_events_armed) return;
    const size_t i = 2 * (size_t)stage + after;
    if (i < g_events.size() && g_events[i] != nullptr) (void)hipEventRecord(g_events[i], st);
}

static hipError_t launch_route(const Geo& g, const moe_shape* s, const RouteArgs& ra, void* ws,
                               const WsLayout& L, hipStream_t st) {
    if (g.rank_route) {
        // the gate with no winners (logits only), then the selection by rank
        RouteArgs lg = ra;
        lg.k = 0;
        if (lg.logits == nullptr) lg.logits = at<float>(ws, L.logits);
        const hipError_t e = g.mfma_gate ? launch_route_mfma(lg, at<uint16_t>(ws, L.gate), device_cu_count(), st)
                                         : launch_route_gate(lg, s->dtype, st);
        if (e != hipSuccess) return e;
        RouteArgs rk = ra;
        rk.logits = lg.logits;
        return launch_route_rank(rk, st);
    }
    if (g.mfma_gate) return launch_route_mfma(ra, at<uint16_t>(ws, L.gate), device_cu_count(), st);
    return launch_route_gate(ra, s->dtype, st);
}

static DispatchArgs dispatch_args(const Geo& g, const moe_shape* s) {
    DispatchArgs a{};
    a.T = g.T;
    a.E = (int)g.E;
    a.k = (int)g.k;
    a.cap = g.cap;
    a.max_rows = g.max_rows;
    a.BT = g.BT;
    a.nblk = g.nblk;
    a.lambda = s->aux_lambda;
    a.row_bytes = g.d * g.esz;
    return a;
}

static hipError_t launch_gemm(const Geo& g, const GemmArgs& ga, int epi, hipStream_t st, bool a_tiled = false) {
    return g.esz == 2 ? launch_ffn_gemm_bf16(ga, epi, g.max_rows, st, a_tiled) : launch_ffn_gemm_f32(ga, epi, st);
}

}  // namespace moe

using namespace moe;

extern "C" {

int64_t moe_capacity(const moe_shape* s) {
    Geo g;
    if (validate(s, &g) != MOE_OK) return -1;
    return g.cap;
}

int64_t moe_max_rows(const moe_shape* s) {
    Geo g;
    if (validate(s, &g) != MOE_OK) return -1;
    return g.max_rows;
}

size_t moe_workspace_size(const moe_shape* s) {
    Geo g;
    if (validate(s, &g) != MOE_OK) return 0;
    return ws_layout(g).total;
}

int64_t moe_workspace_offset(const moe_shape* s, int which) {
    Geo g;
    if (validate(s, &g) != MOE_OK) return -1;
    const WsLayout L = ws_layout(g);
    switch (which) {
        case MOE_WS_PERM: return (int64_t)L.perm;
        case MOE_WS_SLOT: return (int64_t)L.slot;
        case MOE_WS_OFFSETS: return (int64_t)L.offsets;
        case MOE_WS_XPERM: return g.esz == 4 ? (int64_t)L.xperm : -1;
        case MOE_WS_H: return (int64_t)L.h;
        case MOE_WS_OUT: return (int64_t)L.out;
        case MOE_WS_XPT: return (int64_t)L.xpt;
        default: fail(MOE_ERR_SHAPE, "unknown workspace region %d", which); return -1;
    }
}

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL: return "MOE_ERR_NULL";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        default: return "MOE_ERR_UNKNOWN";
    }
}

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

int moe_num_stages(void) { return kNumStages; }

const char* moe_stage_name(int i) { return (i >= 0 && i < kNumStages) ? kStageNames[i] : ""; }

int moe_set_stage_events(void** events, int n_events) {
    if (events == nullptr) return fail(MOE_ERR_NULL, "events is NULL");
    if (n_events != 2 * kNumStages)
        return fail(MOE_ERR_SHAPE, "n_events must be %d (got %d)", 2 * kNumStages, n_events);
    g_events.assign(reinterpret_cast<hipEvent_t*>(events), reinterpret_cast<hipEvent_t*>(events) + n_events);
    g_events_armed = true;
    return MOE_OK;
}

int moe_route(const moe_shape* s, const void* x, const float* Wg, const float* bg, float* logits,
              int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
    Geo g;
    if (int rc = validate(s, &g)) return rc;
    MOE_REQUIRE(x);
    MOE_REQUIRE(Wg);
    MOE_OPTIONAL(bg);
    MOE_OPTIONAL(logits);
    MOE_REQUIRE(topk_idx);
    MOE_REQUIRE(topk_w);
    WsLayout L;
    if (int rc = check_ws(g, ws, ws_bytes, &L)) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    RouteArgs a = route_config(g.T, (int)g.d, (int)g.E, (int)g.k, s->temperature, s->dtype, device_cu_count());
    a.x = x;
    a.Wg = Wg;
    a.bg = bg;
    a.logits = logits;
    a.idx = topk_idx;
    a.w = topk_w;
    MOE_HIP(launch_route(g, s, a, ws, L, st), "route kernel launch");
    return MOE_OK;
}

int moe_route_logits(const moe_shape* s, const float* logits, int32_t* topk_idx, float* topk_w,
                     void* stream) {
    Geo g;
    if (int rc = validate(s, &g)) return rc;
    MOE_REQUIRE(logits);
    MOE_REQUIRE(topk_idx);
    MOE_REQUIRE(topk_w);
    hipStream_t st = static_cast<hipStream_t>(stream);
    RouteArgs a = route_config(g.T, (int)g.d, (int)g.E, (int)g.k, s->temperature, s->dtype, device_cu_count());
    a.logits = const_cast<float*>(logits);
    a.idx = topk_idx;
    a.w = topk_w;
    if (g.rank_route) MOE_HIP(launch_route_rank(a, st), "route_logits kernel launch");
    else MOE_HIP(launch_route_logits(a, st), "route_logits kernel launch");
    return MOE_OK;
}

int moe_dispatch(const moe_shape* s, const void* x, const int32_t* topk_idx, int32_t* routed,
                 int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot, void* x_perm,
                 void* ws, size_t ws_bytes, void* stream) {
    Geo g;
    if (int rc = validate(s, &g)) return rc;
    MOE_REQUIRE(x);
    MOE_REQUIRE(topk_idx);
    MOE_OPTIONAL(routed);
    MOE_REQUIRE(counts);
    MOE_REQUIRE(offsets);
    MOE_REQUIRE(perm);
    MOE_REQUIRE(slot);
    MOE_REQUIRE(x_perm);
    WsLayout L;
    if (int rc = check_ws(g, ws, ws_bytes, &L)) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    DispatchArgs a = dispatch_args(g, s);
    a.idx = topk_idx;
    a.blkhist = at<int32_t>(ws, L.blkhist);
    a.routed = routed;
    a.counts = counts;
    a.offsets = offsets;
    a.perm = perm;
    a.slot = slot;
    a.x = x;
    a.x_perm = x_perm;
    MOE_HIP(launch_hist(a, st), "hist kernel launch");
    MOE_HIP(launch_scatter(a, st), "scatter kernel launch");
    MOE_HIP(launch_gather(a, st), "gather kernel launch");
    return MOE_OK;
}

int moe_dispatch_noalloc(const moe_shape* s, const void* x, const int32_t* topk_idx, int32_t* routed,
                         int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot, void* x_perm,
                         void* stream) {
    Geo g;
    if (int rc = validate(s, &g)) return rc;
    MOE_REQUIRE(x);
    MOE_REQUIRE(topk_idx);
    MOE_OPTIONAL(routed);
    MOE_REQUIRE(counts);
    MOE_REQUIRE(offsets);
    MOE_REQUIRE(perm);
    MOE_REQUIRE(slot);
    MOE_REQUIRE(x_perm);
    const size_t need = sizeof(int32_t) * (size_t)g.nblk * (size_t)g.E;
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_ERR_WORKSPACE,
                    "moe_dispatch_noalloc: the histogram of %d token blocks x %lld experts needs %zu bytes, above "
                    "the %zu-byte static scratch (T=%lld); use moe_dispatch with a workspace",
                    g.nblk, (long long)g.E, need, (size_t)MOE_NOALLOC_SCRATCH_BYTES, (long long)g.T);
    void* sp = nullptr;
    if (int rc = scratch_on_current_device(&sp)) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    DispatchArgs a = dispatch_args(g, s);
    a.idx = topk_idx;
    a.blkhist = static_cast<int32_t*>(sp);   // every entry [b][e] is written by this call's hist launch
    a.routed = routed;
    a.counts = counts;
    a.offsets = offsets;
    a.perm = perm;
    a.slot = slot;
    a.x = x;
    a.x_perm = x_perm;
    MOE_HIP(launch_hist(a, st), "hist kernel launch");
    MOE_HIP(launch_scatter(a, st), "scatter kernel launch");
    MOE_HIP(launch_gather(a, st), "gather kernel launch");
    return MOE_OK;
}

int moe_grouped_ffn(const moe_shape* s, const void* x_perm, const int32_t* offsets, const void* W1,
                    const float* b1, const void* W2, const float* b2, float* out_perm, void* ws,
                    size_t ws_bytes, void* stream) {
    Geo g;
    if (int rc = validate(s, &g)) return rc;
    MOE_REQUIRE(x_perm);
    MOE_REQUIRE(offsets);
    MOE_REQUIRE(W1);
    MOE_REQUIRE(b1);
    MOE_REQUIRE(W2);
    MOE_REQUIRE(b2);
    MOE_REQUIRE(out_perm);
    WsLayout L;
    if (int rc = check_ws(g, ws, ws_bytes, &L)) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    GemmArgs g1{};
    g1.A = x_perm;
    g1.B = W1;
    g1.bias = b1;
    g1.offsets = offsets;
    g1.E = (int)g.E;
    g1.K = (int)g.d;
    g1.N = (int)g.dff;
    g1.out = at<void>(ws, L.h);
    MOE_HIP(launch_gemm(g, g1, EPI_GELU_H, st), "ffn1 kernel launch");
    GemmArgs g2 = g1;
    g2.A = g1.out;
    g2.B = W2;
    g2.bias = b2;
    g2.K = (int)g.dff;
    g2.N = (int)g.d;
    g2.out = out_perm;
    MOE_HIP(launch_gemm(g, g2, EPI_STORE_F32, st), "ffn2 kernel launch");
    return MOE_OK;
}

int moe_combine(const moe_shape* s, const float* out_perm, const int32_t* slot, const float* topk_w,
                float* y, void* stream) {
    Geo g;
    if (int rc = validate(s, &g)) return rc;
    MOE_REQUIRE(out_perm);
    MOE_REQUIRE(slot);
    MOE_REQUIRE(topk_w);
    MOE_REQUIRE(y);
    hipStream_t st = static_cast<hipStream_t>(stream);
    MOE_HIP(launch_combine(g.T, (int)g.d, (int)g.k, out_perm, slot, topk_w, y, st), "combine kernel launch");
    return MOE_OK;
}

int moe_aux_loss(const moe_shape* s, const int32_t* counts, float* aux, void* stream) {
    Geo g;
    if (int rc = validate(s, &g)) return rc;
    MOE_REQUIRE(counts);
    MOE_REQUIRE(aux);
    hipStream_t st = static_cast<hipStream_t>(stream);
    MOE_HIP(launch_aux((int)g.E, g.T, (int)g.k, s->aux_lambda, counts, aux, st), "aux kernel launch");
    return MOE_OK;
}

int moe_route_logits_ex(const moe_shape* s, int mode, const float* logits, const float* noise, float noise_scale,
                        int32_t* topk_idx, float* topk_w, float* noisy_logits, void* stream) {
    Geo g;
    if (int rc = validate(s, &g)) return rc;
    if (mode != MOE_ROUTER_TOPK && mode != MOE_ROUTER_TOP1_FULL)
        return fail(MOE_ERR_SHAPE, "unknown router mode %d", mode);
    if (mode == MOE_ROUTER_TOP1_FULL && g.k != 1)
        return fail(MOE_ERR_SHAPE, "MOE_ROUTER_TOP1_FULL needs k = 1 (got k=%lld)", (long long)g.k);
    if (g.k > kRouteGroupMaxK)
        return fail(MOE_ERR_SHAPE, "the router variants take k <= %d (got k=%lld)", kRouteGroupMaxK, (long long)g.k);
    if (!std::isfinite(noise_scale)) return fail(MOE_ERR_SHAPE, "noise_scale must be finite");
    MOE_REQUIRE(logits);
    MOE_OPTIONAL(noise);
    MOE_REQUIRE(topk_idx);
    MOE_REQUIRE(topk_w);
    MOE_OPTIONAL(noisy_logits);
    hipStream_t st = static_cast<hipStream_t>(stream);
    RouteArgs a = route_config(g.T, (int)g.d, (int)g.E, (int)g.k, s->temperature, s->dtype, device_cu_count());
    a.logits = const_cast<float*>(logits);
    a.idx = topk_idx;
    a.w = topk_w;
    MOE_HIP(launch_route_variant(a, mode, noise, noise_scale, noisy_logits, st), "route variant kernel launch");
    return MOE_OK;
}

int moe_aux_loss_ex(const moe_shape* s, int mode, const int32_t* load, float* aux, void* stream) {
    Geo g;
    if (int rc = validate(s, &g)) return rc;
    if (mode != MOE_LOSS_SHARE && mode != MOE_LOSS_VARIANCE) return fail(MOE_ERR_SHAPE, "unknown loss mode %d", mode);
    MOE_REQUIRE(load);
    MOE_REQUIRE(aux);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (mode == MOE_LOSS_SHARE)
        MOE_HIP(launch_aux((int)g.E, g.T, (int)g.k, s->aux_lambda, load, aux, st), "aux kernel launch");
    else
        MOE_HIP(launch_aux_variance((int)g.E, s->aux_lambda, load, aux, st), "aux variance kernel launch");
    return MOE_OK;
}

struct BwLayout {
    size_t g, h, hgrad, da, dx_perm, dw, ghist, goff, gperm, gslot, dlsel, dlr, wgt, gpart, gpartb, xperm, total;
};

static BwLayout bw_layout(const Geo& g) {
    BwLayout L{};
    size_t p = 0;
    auto take = [&](size_t bytes) {
        const size_t at = p;
        p = align_up(p + (bytes ? bytes : 1));
        return at;
    };
    const size_t R = (size_t)g.max_rows;
    // g, h, GELU'(a) and da in the layer dtype (bf16 operands of the
    // matrix cores in bf16 layers)
    L.g = take((size_t)g.esz * R * g.d);
    L.h = take((size_t)g.esz * R * g.dff);
    L.hgrad = take((size_t)g.esz * R * g.dff);
    L.da = take((size_t)g.esz * R * g.dff);
    L.dx_perm = take(4 * R * g.d);
    const size_t TK = (size_t)(g.T * g.k);
    L.dw = take(4 * TK);
    L.ghist = take(4 * (size_t)g.nblk * g.E);
    L.goff = take(4 * (size_t)(g.E + 1));
    L.gperm = take(4 * TK);
    L.gslot = take(4 * TK);
    L.dlsel = take(4 * TK);
    L.dlr = take(4 * TK);
    L.wgt = take(4 * (size_t)(g.E * g.d));
    const size_t items = (size_t)gate_wgrad_items(g.T, (int)g.k, (int)g.E);
    L.gpart = take(4 * items * g.d);
    L.gpartb = take(4 * items);
    L.xperm = take((size_t)g.esz * R * g.d);   // the rows of x when the caller passes no x_perm
    L.total = p;
    return L;
}

size_t moe_backward_workspace_size(const moe_shape* s) {
    Geo g;
    if (validate(s, &g)) return 0;
    return bw_layout(g).total;
}

int moe_layer_backward(const moe_shape* s, const void* x, const float* Wg, const void* W1, const float* b1,
                       const void* W2, const float* dy, const int32_t* topk_idx, const float* topk_w,
                       const int32_t* slot, const int32_t* offsets, const void* x_perm, const float* out_perm,
                       float* dx, float* dWg, float* dbg, float* dW1, float* db1, float* dW2, float* db2, void* ws,
                       size_t ws_bytes, void* stream) {
    Geo g;
    if (int rc = validate(s, &g)) return rc;
    MOE_REQUIRE(x);
    MOE_REQUIRE(Wg);
    MOE_REQUIRE(W1);
    MOE_REQUIRE(b1);
    MOE_REQUIRE(W2);
    MOE_REQUIRE(dy);
    MOE_REQUIRE(topk_idx);
    MOE_REQUIRE(topk_w);
    MOE_REQUIRE(slot);
    MOE_REQUIRE(offsets);
    MOE_OPTIONAL(x_perm);
    MOE_REQUIRE(out_perm);
    MOE_REQUIRE(dx);
    MOE_REQUIRE(dWg);
    MOE_REQUIRE(dbg);
    MOE_REQUIRE(dW1);
    MOE_REQUIRE(db1);
    MOE_REQUIRE(dW2);
    MOE_REQUIRE(db2);
    const BwLayout L = bw_layout(g);
    if (ws == nullptr) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
    if (misaligned(ws)) return fail(MOE_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
    BackwardArgs b{};
    b.T = g.T;
    b.max_rows = g.max_rows;
    b.d = (int)g.d;
    b.E = (int)g.E;
    b.k = (int)g.k;
    b.dff = (int)g.dff;
    b.tau = s->temperature;
    b.x = x; b.Wg = Wg; b.W1 = W1; b.b1 = b1; b.W2 = W2;
    b.dy = dy; b.topk_idx = topk_idx; b.topk_w = topk_w; b.slot = slot; b.offsets = offsets;
    b.x_perm = x_perm != nullptr ? x_perm : at<void>(ws, L.xperm);
    b.out_perm = out_perm;
    b.dx = dx; b.dWg = dWg; b.dbg = dbg; b.dW1 = dW1; b.db1 = db1; b.dW2 = dW2; b.db2 = db2;
    b.g = at<float>(ws, L.g);
    b.h = at<void>(ws, L.h);
    b.hgrad = at<void>(ws, L.hgrad);
    b.da = at<float>(ws, L.da);
    b.dx_perm = at<float>(ws, L.dx_perm);
    b.dw = at<float>(ws, L.dw);
    b.BT = g.BT;
    b.nblk = g.nblk;
    b.ghist = at<int32_t>(ws, L.ghist);
    b.goff = at<int32_t>(ws, L.goff);
    b.gperm = at<int32_t>(ws, L.gperm);
    b.gslot = at<int32_t>(ws, L.gslot);
    b.dlsel = at<float>(ws, L.dlsel);
    b.dlr = at<float>(ws, L.dlr);
    b.wgt = at<float>(ws, L.wgt);
    b.gpart = at<float>(ws, L.gpart);
    b.gpartb = at<float>(ws, L.gpartb);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (x_perm == nullptr)
        MOE_HIP(launch_gather_slots(g.T, (int)g.k, g.max_rows, g.d * g.esz, x, slot, at<void>(ws, L.xperm), st),
                "backward gather launch");
    MOE_HIP(launch_layer_backward(b, s->dtype, st), "backward kernel launch");
    return MOE_OK;
}

size_t moe_window_state_bytes(int64_t E, int64_t W) {
    if (E < 1 || E > 1024 || W < 1 || W > (int64_t(1) << 20)) return 0;
    return window_state_bytes(E, W);
}

int moe_aux_loss_window(const moe_shape* s, const int32_t* counts, void* state, int64_t W, float* aux, float* pbar,
                        void* stream) {
    Geo g;
    if (int rc = validate(s, &g)) return rc;
    if (W < 1 || W > (int64_t(1) << 20)) return fail(MOE_ERR_SHAPE, "W must be in [1, 2^20] (got %lld)", (long long)W);
    MOE_REQUIRE(counts);
    MOE_REQUIRE(state);
    MOE_REQUIRE(aux);
    MOE_OPTIONAL(pbar);
    hipStream_t st = static_cast<hipStream_t>(stream);
    MOE_HIP(launch_window_aux((int)g.E, W, g.T, (int)g.k, s->aux_lambda, counts, state, aux, pbar, st),
            "window loss kernel launch");
    return MOE_OK;
}

int moe_coactivation(const moe_shape* s, const int32_t* topk_idx, int32_t* H, int32_t* routed, float* stats,
                     void* stream) {
    Geo g;
    if (int rc = validate(s, &g)) return rc;
    MOE_REQUIRE(topk_idx);
    MOE_REQUIRE(H);
    MOE_REQUIRE(routed);
    MOE_OPTIONAL(stats);
    hipStream_t st = static_cast<hipStream_t>(stream);
    MOE_HIP(launch_coactivation(g.T, (int)g.k, (int)g.E, topk_idx, H, routed, stats, device_cu_count(), st),
            "coactivation kernel launch");
    return MOE_OK;
}

int moe_layer_forward(const moe_shape* s, const void* x, const float* Wg, const float* bg, const void* W1,
                      const float* b1, const void* W2, const float* b2, float* y, int32_t* counts,
                      float* aux, int32_t* routed, int32_t* topk_idx, float* topk_w, float* logits,
                      void* ws, size_t ws_bytes, void* stream) {
    struct Disarm {
        ~Disarm() { g_events_armed = false; }
    } disarm;
    Geo g;
    if (int rc = validate(s, &g)) return rc;
    MOE_REQUIRE(x);
    MOE_REQUIRE(Wg);
    MOE_OPTIONAL(bg);
    MOE_REQUIRE(W1);
    MOE_REQUIRE(b1);
    MOE_REQUIRE(W2);
    MOE_REQUIRE(b2);
    MOE_REQUIRE(y);
    MOE_REQUIRE(counts);
    MOE_REQUIRE(aux);
    MOE_OPTIONAL(routed);
    MOE_OPTIONAL(topk_idx);
    MOE_OPTIONAL(topk_w);
    MOE_OPTIONAL(logits);
    WsLayout L;
    if (int rc = check_ws(g, ws, ws_bytes, &L)) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, L.idx);
    float* w = topk_w ? topk_w : at<float>(ws, L.w);

    // 1. gate + top-k + softmax
    RouteArgs ra = route_config(g.T, (int)g.d, (int)g.E, (int)g.k, s->temperature, s->dtype, device_cu_count());
    ra.x = x;
    ra.Wg = Wg;
    ra.bg = bg;
    ra.logits = logits;
    ra.idx = idx;
    ra.w = w;
    stage_event(0, 0, st);
    MOE_HIP(launch_route(g, s, ra, ws, L, st), "route kernel launch");
    stage_event(0, 1, st);

    // 2. dispatch
    DispatchArgs da = dispatch_args(g, s);
    da.idx = idx;
    da.blkhist = at<int32_t>(ws, L.blkhist);
    da.routed = routed;
    da.counts = counts;
    da.offsets = at<int32_t>(ws, L.offsets);
    da.perm = at<int32_t>(ws, L.perm);
    da.slot = at<int32_t>(ws, L.slot);
    da.aux = aux;
    da.x = x;
    da.x_perm = g.esz == 4 ? at<void>(ws, L.xperm) : nullptr;   // bf16: the tile copy x_pt instead
    stage_event(1, 0, st);
    MOE_HIP(launch_hist(da, st), "hist kernel launch");
    stage_event(1, 1, st);
    stage_event(2, 0, st);
    MOE_HIP(launch_scatter(da, st), "scatter kernel launch");
    stage_event(2, 1, st);
    // bf16: x_perm only in the tile layout GEMM1 loads in contiguous KiBs
    // (moe_layer_backward copies the row-major rows itself); fp32: row-major
    const bool tiled = g.esz == 2;
    stage_event(3, 0, st);
    if (tiled) MOE_HIP(launch_gather_tiled(da, at<uint16_t>(ws, L.xpt), (int)g.d, st), "gather kernel launch");
    else MOE_HIP(launch_gather(da, st), "gather kernel launch");
    stage_event(3, 1, st);

    // 3. grouped FFN over the expert-contiguous rows
    GemmArgs g1{};
    g1.A = tiled ? at<void>(ws, L.xpt) : da.x_perm;
    g1.B = W1;
    g1.bias = b1;
    g1.offsets = da.offsets;
    g1.E = (int)g.E;
    g1.K = (int)g.d;
    g1.N = (int)g.dff;
    g1.out = at<void>(ws, L.h);
    stage_event(4, 0, st);
    MOE_HIP(launch_gemm(g, g1, EPI_GELU_H, st, tiled), "ffn1 kernel launch");
    stage_event(4, 1, st);
    GemmArgs g2 = g1;
    g2.A = g1.out;
    g2.B = W2;
    g2.bias = b2;
    g2.K = (int)g.dff;
    g2.N = (int)g.d;
    g2.out = at<float>(ws, L.out);
    stage_event(5, 0, st);
    MOE_HIP(launch_gemm(g, g2, EPI_STORE_F32, st), "ffn2 kernel launch");
    stage_event(5, 1, st);

    // 4. weighted sum back to token order (overwrites y)
    stage_event(6, 0, st);
    MOE_HIP(launch_combine(g.T, (int)g.d, (int)g.k, at<float>(ws, L.out), da.slot, w, y, st),
            "combine kernel launch");
    stage_event(6, 1, st);
    return MOE_OK;
}

}  // extern "C"
