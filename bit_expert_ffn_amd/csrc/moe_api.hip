// C ABI of libmoe_ffn: argument validation, workspace layout and launches.
// The operations are defined in include/moe_ffn.h with their sources.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>

#include "../../include/moe_ffn.h"
#include "moe_internal.h"

namespace moe {

static thread_local char g_err[512] = "";

// Bound of every kernel wait (polls); negative = the default.
static std::atomic<long> g_wait_polls{-1};

// Compute units of the current device (the one-token kernel's down tiling
// depends on it), cached per device.
static hipError_t device_cus(int* out) {
    static std::mutex mu;
    static std::map<int, int> cus;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cus.find(dev);
    if (it == cus.end()) {
        int n = 0;
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        it = cus.emplace(dev, n).first;
    }
    *out = it->second;
    return hipSuccess;
}
long wait_polls() {
    const long v = g_wait_polls.load(std::memory_order_relaxed);
    return v < 0 ? kDefaultWaitPolls : v;
}

// The matrix-core path addresses the fp16 activation planes [2][T][H] and the
// `a` planes [2][rows][FFmax] with 32-bit byte offsets: the largest T whose
// offsets stay below 2^32 (with a 4 KiB margin for the last chunk's reads).
static int64_t prefill_max_tokens(int k, int H, int FF, int FFs) {
    const int64_t lim = ((int64_t)1 << 32) - 4096;
    const int64_t ffmax = FFs > FF ? FFs : FF;
    const int64_t per_x = (int64_t)4 * H;                         // 2 planes x 2 bytes
    const int64_t per_a = (int64_t)4 * ffmax * (k + (FFs ? 1 : 0));   // 2 planes x 2 bytes per row, k (+1) rows
    const int64_t t1 = lim / per_x, t2 = lim / per_a;
    return t1 < t2 ? t1 : t2;
}

static moe_status fail(moe_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Bump {
    size_t off = 0;
    size_t take(size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    }
};

SmallLayout small_layout(int T, int k, int E, int H, int FF, int FFs, int qtype) {
    SmallLayout L{};
    Bump b;
    const size_t n = (size_t)T * k;
    const size_t s1 = decode_sync_bytes(kSmallT * k + kSmallT);
    const size_t sw = window_sync_bytes(k, window_shape(H, FF, FFs, qtype, MOE_F32, kSmallT, k).n_chunks);
    L.sync = b.take(s1 > sw ? s1 : sw);
    L.a = b.take((size_t)kSmallT * k * FF * 4);
    L.as = b.take((size_t)kSmallT * FFs * 4);
    L.d = b.take((size_t)(kSmallT * k + kSmallT) * H * 4);
    L.ids = b.take(n * 4);
    L.w = b.take(n * 4);
    L.logits = b.take((size_t)T * E * 4);
    L.total = b.off;
    return L;
}

size_t small_fixed_bytes(int k, int H, int FF, int FFs, int qtype) {
    return small_layout(0, k, 1, H, FF, FFs, qtype).ids;
}

// Workspace of moe_layer_forward_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes its name to a
// kernel (on the host the name is only a stand-in): its device address comes
// from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static hipError_t scratch_address(void** out) {
    static std::mutex mu;
    static std::map<int, void*> addr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    auto it = addr.find(dev);
    if (it == addr.end()) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        it = addr.emplace(dev, p).first;
    }
    *out = it->second;
    return hipSuccess;
}

// Zero-fill of n16 16-byte words (a kernel rather than a memset node, so that
// a captured graph replays it correctly).
__global__ void __launch_bounds__(256) zero_fill_kernel(uint4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace moe

using namespace moe;

static moe_status check_expert(const moe_expert_desc* d, const char* what) {
    if (!d) return fail(MOE_ERR_INVALID_ARG, "%s: descriptor is NULL", what);
    const int qk = codes_per_block(d->qtype);
    if (qk == 0) return fail(MOE_ERR_INVALID_ARG, "%s: unknown qtype %d", what, d->qtype);
    if (d->hidden <= 0 || d->ff <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: hidden and ff must be > 0", what);
    if (d->hidden % qk || d->ff % qk)
        return fail(MOE_ERR_INVALID_ARG, "%s: hidden (%d) and ff (%d) must be multiples of %d", what, d->hidden,
                    d->ff, qk);
    if (d->act != MOE_ACT_SWIGLU && d->act != MOE_ACT_GEGLU_TANH)
        return fail(MOE_ERR_UNSUPPORTED, "%s: activation %d not supported", what, d->act);
    if (!isfinite(d->zero_point)) return fail(MOE_ERR_INVALID_ARG, "%s: zero_point is not finite", what);
    if (fabsf(d->zero_point) > 64.f || d->zero_point * 2.f != floorf(d->zero_point * 2.f))
        return fail(MOE_ERR_UNSUPPORTED, "%s: zero_point %g is not a multiple of 0.5 in [-64, 64]", what,
                    (double)d->zero_point);
    if (d->hidden / qk > kMaxBlocksPerRow || d->ff / qk > kMaxBlocksPerRow)
        return fail(MOE_ERR_UNSUPPORTED, "%s: more than %d blocks per row", what, kMaxBlocksPerRow);
    return MOE_OK;
}

static moe_status check_layer(const moe_layer_desc* d) {
    if (!d) return fail(MOE_ERR_INVALID_ARG, "layer descriptor is NULL");
    moe_status s = check_expert(&d->expert, "layer");
    if (s != MOE_OK) return s;
    if (d->n_experts < 1 || d->n_experts > kMaxE)
        return fail(MOE_ERR_UNSUPPORTED, "n_experts %d outside [1, %d]", d->n_experts, kMaxE);
    if (d->top_k < 1 || d->top_k > d->n_experts)
        return fail(MOE_ERR_INVALID_ARG, "top_k %d outside [1, n_experts=%d]", d->top_k, d->n_experts);
    if (d->top_k > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "top_k %d above %d", d->top_k, kMaxK);
    if (d->renormalize != 0 && d->renormalize != 1) return fail(MOE_ERR_INVALID_ARG, "renormalize must be 0 or 1");
    const int qk = codes_per_block(d->expert.qtype);
    if (d->shared_ff < 0 || d->shared_ff % qk)
        return fail(MOE_ERR_INVALID_ARG, "shared_ff %d must be >= 0 and a multiple of %d", d->shared_ff, qk);
    if (d->shared_ff / qk > kMaxBlocksPerRow) return fail(MOE_ERR_UNSUPPORTED, "shared_ff too large");
    return MOE_OK;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

extern "C" {

const char* moe_status_str(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    }
    return "unknown moe_status";
}

const char* moe_last_error(void) { return g_err; }

size_t moe_expert_blob_bytes(const moe_expert_desc* d) {
    if (check_expert(d, "blob") != MOE_OK) return 0;
    const int qk = codes_per_block(d->qtype);
    return (size_t)3 * ((size_t)d->hidden * d->ff / qk) * kBlockBytes;
}

size_t moe_layer_workspace_bytes(const moe_layer_desc* d, int32_t T) {
    if (check_layer(d) != MOE_OK || T < 0) return 0;
    if (T <= kSmallT)
        return small_layout(T, d->top_k, d->n_experts, d->expert.hidden, d->expert.ff, d->shared_ff, d->expert.qtype)
            .total;
    return large_layout(T, d->top_k, d->n_experts, d->expert.hidden, d->expert.ff, d->shared_ff, d->expert.qtype)
        .total;
}

size_t moe_expert_workspace_bytes(const moe_expert_desc* d, int32_t T) {
    if (check_expert(d, "expert") != MOE_OK || T < 0) return 0;
    if (T <= kSmallT) return small_layout(T, 1, 1, d->hidden, d->ff, 0, d->qtype).total;
    return large_layout(T, 1, 1, d->hidden, d->ff, 0, d->qtype).total;
}

moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renormalize, int32_t* ids,
                          float* weights, void* stream) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T < 0");
    if (E < 1 || E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E %d outside [1, %d]", E, kMaxE);
    if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "k %d outside [1, E=%d]", k, E);
    if (k > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "k %d above %d", k, kMaxK);
    if (renormalize != 0 && renormalize != 1) return fail(MOE_ERR_INVALID_ARG, "renormalize must be 0 or 1");
    if (T == 0) return MOE_OK;
    if (!logits || !ids || !weights) return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(weights, 4))
        return fail(MOE_ERR_INVALID_ARG, "pointers must be 4-byte aligned");
    hipError_t e = launch_route_topk(logits, T, E, k, renormalize, ids, weights, (hipStream_t)stream);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "route launch: %s", hipGetErrorString(e));
    return MOE_OK;
}

static moe_status run_layer(int T, int E, int k, int renorm, const moe_expert_desc& ed, int FFs,
                            const void* const* table, const void* single, const void* shared, const void* x,
                            int x_dtype, const float* logits, const moe_layer_opts* opts, float* y, int32_t* ids_out,
                            float* w_out, void* ws, size_t ws_bytes, hipStream_t s, bool identity,
                            StageMarks* marks = nullptr) {
    char* wsb = (char*)ws;
    LayerOpts o;
    o.act = ed.act;
    const moe_router* router = nullptr;
    float* logits_out = nullptr;
    if (opts) {
        o.down_scale = opts->down_scale;
        o.ids_in = opts->ids_in;
        o.w_in = opts->w_in;
        router = opts->router;
        logits_out = opts->logits_out;
    }
    // The router, when it runs inside the call, writes the logits the layer
    // kernels read (into the caller's buffer or the workspace).
    auto run_router = [&](size_t ws_logits) -> hipError_t {
        if (!router) return hipSuccess;
        float* lg = logits_out ? logits_out : (float*)(wsb + ws_logits);
        stage_mark(marks, s);
        hipError_t e = launch_router(router->weight, router->in_scale, router->norm, router->eps, E, ed.hidden, x,
                                     x_dtype, T, lg, s);
        logits = lg;
        return e;
    };
    if (T <= kSmallT) {
        const SmallLayout L = small_layout(T, k, E, ed.hidden, ed.ff, FFs, ed.qtype);
        if (ws_bytes < L.total)
            return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, L.total);
        hipError_t e;
        if (T == 1) {
            int n_cu = 0;
            e = device_cus(&n_cu);
            if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "device query: %s", hipGetErrorString(e));
            const GemvShape g = gemv_shape(ed.hidden, ed.ff, FFs, ed.qtype, ed.zero_point, T, k, n_cu);
            if (g.lds_bytes > 128 * 1024)
                return fail(MOE_ERR_UNSUPPORTED, "decode tile needs %zu bytes of LDS", g.lds_bytes);
            e = run_router(L.logits);
            if (e == hipSuccess)
                e = launch_decode_layer(g, table, single, shared, x, x_dtype, logits, T, E, k, renorm,
                                        identity ? 1 : 0, o, ids_out, w_out, L, wsb, y, s, marks);
        } else {
            const WindowShape g = window_shape(ed.hidden, ed.ff, FFs, ed.qtype, x_dtype, T, k);
            if (g.lds_bytes > 148 * 1024)
                return fail(MOE_ERR_UNSUPPORTED, "verify window needs %zu bytes of LDS", g.lds_bytes);
            e = run_router(L.logits);
            if (e == hipSuccess)
                e = launch_window_layer(g, table, single, shared, x, x_dtype, logits, T, E, k, renorm,
                                        identity ? 1 : 0, o, ed.qtype, ed.zero_point, ed.hidden, ed.ff, FFs, ids_out,
                                        w_out, L, wsb, y, s, marks);
        }
        if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "decode launch: %s", hipGetErrorString(e));
        return MOE_OK;
    }
    const int64_t t_max = prefill_max_tokens(k, ed.hidden, ed.ff, FFs);
    if (T > t_max)
        return fail(MOE_ERR_UNSUPPORTED, "T = %d above %lld, the largest the 32-bit offsets of the matrix-core path "
                    "address at this shape", T, (long long)t_max);
    const LargeLayout L = large_layout(T, k, E, ed.hidden, ed.ff, FFs, ed.qtype);
    if (ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, L.total);
    hipError_t e = run_router(L.logits);
    if (e == hipSuccess)
        e = launch_prefill_layer(table, single, shared, ed.qtype, ed.zero_point, ed.hidden, ed.ff, FFs, x, x_dtype,
                                 logits, T, E, k, renorm, identity ? 1 : 0, o, ids_out, w_out, L, wsb, y, s, marks);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "prefill launch: %s", hipGetErrorString(e));
    return MOE_OK;
}

moe_status moe_expert_ffn(const moe_expert_desc* desc, const void* blob, const void* x, int32_t x_dtype, int32_t T,
                          float* y, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_expert(desc, "moe_expert_ffn");
    if (st != MOE_OK) return st;
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T < 0");
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "unknown x_dtype %d", x_dtype);
    if (T == 0) return MOE_OK;
    if (T > kSmallT && T > prefill_max_tokens(1, desc->hidden, desc->ff, 0))
        return fail(MOE_ERR_UNSUPPORTED, "T = %d above %lld, the largest the matrix-core path addresses", T,
                    (long long)prefill_max_tokens(1, desc->hidden, desc->ff, 0));
    if (!blob || !x || !y || !ws) return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(blob, 16) || !aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 256))
        return fail(MOE_ERR_INVALID_ARG, "blob, x and y must be 16-byte aligned and ws 256-byte aligned");
    const size_t need = moe_expert_workspace_bytes(desc, T);
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
    return run_layer(T, 1, 1, 1, *desc, 0, nullptr, blob, nullptr, x, x_dtype, nullptr, nullptr, y, nullptr, nullptr,
                     ws, ws_bytes, (hipStream_t)stream, true);
}

static moe_status check_router(const moe_router* r, int H) {
    if (!r->weight) return fail(MOE_ERR_INVALID_ARG, "router weight is NULL");
    if (!aligned(r->weight, 16) || (r->in_scale && !aligned(r->in_scale, 16)))
        return fail(MOE_ERR_INVALID_ARG, "router weight and in_scale must be 16-byte aligned");
    if (r->norm != 0 && r->norm != 1) return fail(MOE_ERR_INVALID_ARG, "router norm must be 0 or 1");
    if (!isfinite(r->eps) || r->eps < 0.f) return fail(MOE_ERR_INVALID_ARG, "router eps must be finite and >= 0");
    if (H % 32) return fail(MOE_ERR_INVALID_ARG, "router: H must be a multiple of 32");
    return MOE_OK;
}

static moe_status layer_forward_checked(const moe_layer_desc* desc, const void* const* expert_table,
                                        const void* shared_blob, const void* x, int32_t x_dtype, const float* logits,
                                        int32_t T, float* y, int32_t* ids_out, float* w_out, void* ws,
                                        size_t ws_bytes, void* stream, StageMarks* marks,
                                        const moe_layer_opts* opts = nullptr) {
    moe_status st = check_layer(desc);
    if (st != MOE_OK) return st;
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T < 0");
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "unknown x_dtype %d", x_dtype);
    if ((desc->shared_ff > 0) != (shared_blob != nullptr))
        return fail(MOE_ERR_INVALID_ARG, "shared_blob must be non-NULL exactly when shared_ff > 0");
    if (T == 0) return MOE_OK;
    if (T > kSmallT && T > prefill_max_tokens(desc->top_k, desc->expert.hidden, desc->expert.ff, desc->shared_ff))
        return fail(MOE_ERR_UNSUPPORTED, "T = %d above %lld, the largest the matrix-core path addresses at this shape",
                    T, (long long)prefill_max_tokens(desc->top_k, desc->expert.hidden, desc->expert.ff,
                                                     desc->shared_ff));
    const bool routed = opts && opts->ids_in;
    const bool router = opts && opts->router;
    if (opts) {
        if (routed && router) return fail(MOE_ERR_INVALID_ARG, "ids_in and router are exclusive");
        if (routed != (opts->w_in != nullptr)) return fail(MOE_ERR_INVALID_ARG, "ids_in and w_in come together");
        if (router && logits) return fail(MOE_ERR_INVALID_ARG, "logits must be NULL when the router computes them");
        if (!router && opts->logits_out) return fail(MOE_ERR_INVALID_ARG, "logits_out needs the router");
        if ((opts->ids_in && !aligned(opts->ids_in, 4)) || (opts->w_in && !aligned(opts->w_in, 4)) ||
            (opts->down_scale && !aligned(opts->down_scale, 4)) || (opts->logits_out && !aligned(opts->logits_out, 4)))
            return fail(MOE_ERR_INVALID_ARG, "misaligned option pointer (4 B)");
        if (router) {
            moe_status rs = check_router(opts->router, desc->expert.hidden);
            if (rs != MOE_OK) return rs;
        }
    }
    if (!expert_table || !x || (!logits && !routed && !router) || !y || !ws)
        return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(x, 16) || !aligned(y, 16) || (logits && !aligned(logits, 4)) || !aligned(ws, 256) ||
        !aligned(expert_table, 8) || (shared_blob && !aligned(shared_blob, 16)) || (ids_out && !aligned(ids_out, 4)) ||
        (w_out && !aligned(w_out, 4)))
        return fail(MOE_ERR_INVALID_ARG, "misaligned pointer (x, y, blobs: 16 B; ws: 256 B)");
    const size_t need = moe_layer_workspace_bytes(desc, T);
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
    return run_layer(T, desc->n_experts, desc->top_k, desc->renormalize, desc->expert, desc->shared_ff, expert_table,
                     nullptr, shared_blob, x, x_dtype, routed ? nullptr : logits, opts, y, ids_out, w_out, ws,
                     ws_bytes, (hipStream_t)stream, false, marks);
}

moe_status moe_layer_forward_ex(const moe_layer_desc* desc, const moe_layer_opts* opts,
                                const void* const* expert_table, const void* shared_blob, const void* x,
                                int32_t x_dtype, const float* logits, int32_t T, float* y, int32_t* ids_out,
                                float* w_out, void* ws, size_t ws_bytes, void* stream) {
    return layer_forward_checked(desc, expert_table, shared_blob, x, x_dtype, logits, T, y, ids_out, w_out, ws,
                                 ws_bytes, stream, nullptr, opts);
}

moe_status moe_router_logits(const moe_router* router, int32_t E, int32_t H, const void* x, int32_t x_dtype,
                             int32_t T, float* logits, void* stream) {
    if (!router) return fail(MOE_ERR_INVALID_ARG, "router is NULL");
    if (E < 1 || H < 32 || T < 0) return fail(MOE_ERR_INVALID_ARG, "E >= 1, H >= 32 and T >= 0 required");
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "unknown x_dtype %d", x_dtype);
    moe_status st = check_router(router, H);
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (!x || !logits) return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(x, 16) || !aligned(logits, 4)) return fail(MOE_ERR_INVALID_ARG, "x must be 16-byte aligned");
    hipError_t e = launch_router(router->weight, router->in_scale, router->norm, router->eps, E, H, x, x_dtype, T,
                                 logits, (hipStream_t)stream);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "router launch: %s", hipGetErrorString(e));
    return MOE_OK;
}

moe_status moe_layer_forward(const moe_layer_desc* desc, const void* const* expert_table, const void* shared_blob,
                             const void* x, int32_t x_dtype, const float* logits, int32_t T, float* y,
                             int32_t* ids_out, float* w_out, void* ws, size_t ws_bytes, void* stream) {
    return layer_forward_checked(desc, expert_table, shared_blob, x, x_dtype, logits, T, y, ids_out, w_out, ws,
                                 ws_bytes, stream, nullptr);
}

moe_status moe_layer_forward_timed(const moe_layer_desc* desc, const void* const* expert_table,
                                   const void* shared_blob, const void* x, int32_t x_dtype, const float* logits,
                                   int32_t T, float* y, int32_t* ids_out, float* w_out, void* ws, size_t ws_bytes,
                                   void* stream, void* const* events, int32_t n_events, int32_t* n_kernels) {
    if (n_events < 0 || (n_events > 0 && !events))
        return fail(MOE_ERR_INVALID_ARG, "events must hold n_events >= 0 entries");
    for (int i = 0; i < n_events; ++i)
        if (!events[i]) return fail(MOE_ERR_INVALID_ARG, "events[%d] is NULL", i);
    StageMarks m;
    m.ev = (const hipEvent_t*)events;
    m.n = n_events;
    if (n_kernels) *n_kernels = 0;
    moe_status st = layer_forward_checked(desc, expert_table, shared_blob, x, x_dtype, logits, T, y, ids_out, w_out, ws,
                                          ws_bytes, stream, &m);
    if (st != MOE_OK) return st;
    if (m.err != hipSuccess) return fail(MOE_ERR_DEVICE, "hipEventRecord: %s", hipGetErrorString(m.err));
    if (n_kernels) *n_kernels = m.next > 0 ? m.next - 1 : 0;
    return MOE_OK;
}

moe_status moe_dequant_matrix(const moe_expert_desc* desc, const void* blob, int32_t m, float* out, void* stream) {
    moe_status st = check_expert(desc, "moe_dequant_matrix");
    if (st != MOE_OK) return st;
    if (m < 0 || m > 2) return fail(MOE_ERR_INVALID_ARG, "matrix index %d outside [0, 2]", m);
    if (!blob || !out) return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(blob, 16) || !aligned(out, 4)) return fail(MOE_ERR_INVALID_ARG, "misaligned pointer");
    const int qk = codes_per_block(desc->qtype);
    const int H = desc->hidden, FF = desc->ff;
    const int rows = m == 2 ? H : FF, cols = m == 2 ? FF : H;
    const size_t mat_bytes = (size_t)FF * (H / qk) * kBlockBytes;   // gate and up are the same size
    hipError_t e = launch_dequant(blob, desc->qtype, desc->zero_point, rows, cols, (size_t)m * mat_bytes, out,
                                  (hipStream_t)stream);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "dequant launch: %s", hipGetErrorString(e));
    return MOE_OK;
}

moe_status moe_layer_forward_noalloc(const moe_layer_desc* desc, const void* const* expert_table,
                                     const void* shared_blob, const void* x, int32_t x_dtype, const float* logits,
                                     int32_t T, float* y, int32_t* ids_out, float* w_out, void* stream) {
    moe_status st = check_layer(desc);
    if (st != MOE_OK) return st;
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T < 0");
    if (T > kSmallT)
        return fail(MOE_ERR_UNSUPPORTED, "moe_layer_forward_noalloc serves T <= %d (decode and verify windows), got %d",
                    kSmallT, T);
    const size_t need = moe_layer_workspace_bytes(desc, T);
    if (need > kScratchBytes)
        return fail(MOE_ERR_WORKSPACE, "this shape needs %zu bytes of workspace, above the %zu-byte device array of "
                    "moe_layer_forward_noalloc", need, kScratchBytes);
    if (T == 0) return layer_forward_checked(desc, expert_table, shared_blob, x, x_dtype, logits, T, y, ids_out, w_out,
                                             nullptr, 0, stream, nullptr);
    void* ws = nullptr;
    hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetSymbolAddress: %s", hipGetErrorString(e));
    // The array keeps the last call's contents: its shared region is cleared
    // before this call uses it (a failed earlier call may have left it set).
    const size_t fixed = small_fixed_bytes(desc->top_k, desc->expert.hidden, desc->expert.ff, desc->shared_ff,
                                           desc->expert.qtype);
    const size_t n16 = fixed / 16;
    const unsigned blocks = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
    hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint4*)ws, n16);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "zero-fill launch: %s", hipGetErrorString(e));
    return layer_forward_checked(desc, expert_table, shared_blob, x, x_dtype, logits, T, y, ids_out, w_out, ws,
                                 kScratchBytes, stream, nullptr);
}

int64_t moe_max_tokens(const moe_layer_desc* desc) {
    if (check_layer(desc) != MOE_OK) return 0;
    return prefill_max_tokens(desc->top_k, desc->expert.hidden, desc->expert.ff, desc->shared_ff);
}

moe_status moe_workspace_check(const moe_layer_desc* desc, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_layer(desc);
    if (st != MOE_OK) return st;
    if (!ws || !aligned(ws, 256)) return fail(MOE_ERR_INVALID_ARG, "ws must be a 256-byte aligned device pointer");
    const size_t fixed = small_fixed_bytes(desc->top_k, desc->expert.hidden, desc->expert.ff, desc->shared_ff,
                                           desc->expert.qtype);
    if (ws_bytes < fixed) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, fixed);
    hipStream_t s = (hipStream_t)stream;
    int word = 0;
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess)
        e = hipMemcpy(&word, (const char*)ws + (size_t)kErrWord * sizeof(int), sizeof(int), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "workspace check: %s", hipGetErrorString(e));
    if (word == 0) return MOE_OK;
    // The failed call may have left any of the shared words set: return the
    // whole fixed region (synchronisation words, `a`, d) to zero.
    e = hipMemsetAsync(ws, 0, fixed, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "workspace reset: %s", hipGetErrorString(e));
    return fail(MOE_ERR_DEVICE, "a layer call on this workspace failed (error bits 0x%x:%s%s); its outputs were "
                "NaN; the workspace is reset", word, (word & kErrTimeout) ? " a bounded wait gave up" : "",
                (word & kErrBadId) ? " an expert id outside [0, E)" : "");
}

void moe_debug_set_wait_limit(int64_t polls) { g_wait_polls.store(polls < 0 ? -1 : (long)polls); }

moe_status moe_validate_table(const void* const* expert_table, int32_t E, void* stream) {
    if (!expert_table || E < 1) return fail(MOE_ERR_INVALID_ARG, "NULL table or E < 1");
    void** host = (void**)malloc(sizeof(void*) * (size_t)E);
    if (!host) return fail(MOE_ERR_DEVICE, "host allocation failed");
    hipError_t e = hipMemcpyAsync(host, expert_table, sizeof(void*) * (size_t)E, hipMemcpyDeviceToHost,
                                  (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) {
        free(host);
        return fail(MOE_ERR_DEVICE, "table copy: %s", hipGetErrorString(e));
    }
    for (int i = 0; i < E; ++i)
        if (!host[i]) {
            free(host);
            return fail(MOE_ERR_INVALID_ARG, "expert_table[%d] is NULL", i);
        }
    free(host);
    return MOE_OK;
}

}  // extern "C"
