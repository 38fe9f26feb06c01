// C ABI of libcoli_moe: argument checks, workspace carving and the launch
// sequence of each call (include/coli_moe.h documents every entry point).
#include <algorithm>
#include <exception>
#include <mutex>
#include <new>
#include <string>

#include "common.h"
#include "gemm.h"
#include "layer.h"
#include "quant.h"

namespace coli {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

coli_status fail(coli_status code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

coli_status hip_fail(hipError_t err, const char* what) {
    g_last_error = std::string(what) + ": " + hipGetErrorString(err);
    return COLI_EHIP;
}

coli_status check_shape(const coli_moe_shape* s) {
    if (!s) return fail(COLI_EINVAL, "shape is NULL");
    if (s->hidden <= 0 || s->inter <= 0 || s->hidden % kBlock || s->inter % kBlock)
        return fail(COLI_EINVAL, "hidden and inter must be positive multiples of 32");
    if (s->group != 0 && s->group != 64) return fail(COLI_EUNSUPPORTED, "group must be 0 or 64");
    if (s->group == 64 && (s->hidden % 64 || s->inter % 64))
        return fail(COLI_EINVAL, "group 64 needs hidden and inter multiples of 64");
    if (s->n_routed < 1 || s->n_routed > 1024) return fail(COLI_EUNSUPPORTED, "n_routed must be in [1, 1024]");
    if (s->n_shared != 0 && s->n_shared != 1) return fail(COLI_EUNSUPPORTED, "n_shared must be 0 or 1");
    if (s->top_k < 1 || s->top_k > 32 || s->top_k > s->n_routed)
        return fail(COLI_EUNSUPPORTED, "top_k must be in [1, min(32, n_routed)]");
    if (s->hidden > 16384) return fail(COLI_EUNSUPPORTED, "hidden must be <= 16384");
    if (s->inter > 4096) return fail(COLI_EUNSUPPORTED, "inter must be <= 4096");
    if (!(s->routed_scale == s->routed_scale) || s->routed_scale > 3.4e38f || s->routed_scale < -3.4e38f)
        return fail(COLI_EINVAL, "routed_scale must be finite");
    if (!(s->topp >= 0.f && s->topp <= 1.f)) return fail(COLI_EINVAL, "topp must be in [0, 1]");
    if (s->wbits != 0 && s->wbits != 4 && s->wbits != 8) return fail(COLI_EUNSUPPORTED, "wbits must be 4 or 8");
    return COLI_OK;
}

// Workspace carving: every region 256-byte aligned, in a fixed order.
WsLayout ws_layout(const coli_moe_shape* s, int32_t T, int32_t path) {
    (void)path;
    WsLayout W;
    const size_t E = (size_t)s->n_routed, k = (size_t)s->top_k, H = (size_t)s->hidden,
                 I = (size_t)s->inter, n = (size_t)T * k, R = n + (size_t)T;
    size_t o = 0;
    auto take = [&o](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
    W.logits = take((size_t)T * E * 4);
    W.idx = take(n * 4);
    W.w = take(n * 4);
    W.counts = take(E * 4);
    W.offsets = take((E + 1) * 4);
    W.perm = take(n * 4);
    W.unique = take(E * 4);
    W.n_unique = take(4);
    W.n_items = take(4);
    W.union_ws = take(union_ws_bytes(T, (int32_t)k, (int32_t)E));
    W.items = take((size_t)std::max<int64_t>(E + 1, split_items_bound(E, T, k, true)) * sizeof(WorkItem));
    W.rows_tok = take(R * 4);
    W.rows_out = take(R * 4);
    W.xplanes = take((size_t)T * (H / kBlock) * kWordsPerBlock * 4);
    W.xscale = take((size_t)T * (H / kBlock) * 4);
    W.hplanes = take(R * (I / kBlock) * kWordsPerBlock * 4);
    W.hscale = take(R * (I / kHBlock) * 4);
    W.y_rows = take(R * H * 4);
    W.phase = take(E);
    W.codes = take(E * 8);
    W.scores = take(E * 4);
    // bf16 MFMA path
    const size_t max_items = std::min<size_t>(E, n) + 1;
    W.max_tiles = gemm_tiles_max((int32_t)R, (int32_t)max_items);
    W.tiles = take(W.max_tiles * 8);
    W.n_tiles = take(4);
    W.gv_items = take(max_items * sizeof(WorkItem));
    W.n_gv = take(4);
    W.xb = take((size_t)T * H * 2);
    W.sx = take((size_t)T * (H / 64) * 4);
    W.hb = take(R * I * 2);
    W.sh = take(R * (I / 64) * 4);
    W.bytes = o;
    return W;
}

// ------------------------------------------------ allocation-free layer call
// coli_moe_layer_fwd_noalloc runs on this file-scope device array instead of a
// caller's workspace. Every GPU the library runs on holds its own copy until
// the process ends. In host code `scratch` names a host-side stand-in, never
// the device memory: the device address is looked up once per device with
// hipGetSymbolAddress and only that pointer is handed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static uint8_t* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the calling thread's current device,
// looked up on the first call there.
static coli_status scratch_on_current_device(uint8_t** out) {
    int dev = -1;
    COLI_CHECK_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(COLI_EUNSUPPORTED, "noalloc: device ordinal above 63");
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "noalloc: hipGetSymbolAddress(scratch)");
        if (!p) return fail(COLI_EHIP, "noalloc: no device address for the scratch array");
        g_scratch_ptr[dev] = (uint8_t*)p;
    }
    *out = g_scratch_ptr[dev];
    return COLI_OK;
}

}  // namespace coli

using namespace coli;

#define COLI_GUARD_BEGIN try {
#define COLI_GUARD_END                                                          \
    }                                                                           \
    catch (const std::bad_alloc&) { return fail(COLI_ENOMEM, "host allocation failed"); } \
    catch (const std::exception& ex) { return fail(COLI_EINVAL, ex.what()); }  \
    catch (...) { return fail(COLI_EINVAL, "unknown error"); }

extern "C" {

const char* coli_last_error(void) { return g_last_error.c_str(); }

const char* coli_version(void) { return "coli_moe 0.1 (gfx950)"; }

coli_status coli_expert_blob_layout(const coli_moe_shape* shape, size_t off[6], size_t* blob_bytes) {
    COLI_GUARD_BEGIN
    coli_status st = check_shape(shape);
    if (st) return st;
    if (!off || !blob_bytes) return fail(COLI_EINVAL, "off or blob_bytes is NULL");
    const BlobLayout L = blob_layout(shape->hidden, shape->inter, shape->group, shape->wbits);
    off[0] = L.gate_q; off[1] = L.up_q; off[2] = L.down_q;
    off[3] = L.gate_s; off[4] = L.up_s; off[5] = L.down_s;
    *blob_bytes = L.bytes;
    return COLI_OK;
    COLI_GUARD_END
}

coli_status coli_quantize_int4(const float* d_w, int64_t rows, int64_t cols, int32_t group,
                               uint8_t* d_q, float* d_s, void* stream) {
    COLI_GUARD_BEGIN
    if (rows < 0 || cols <= 0 || (cols & 1)) return fail(COLI_EINVAL, "quantize: rows >= 0, cols even and > 0");
    if (group != 0 && group != 64) return fail(COLI_EUNSUPPORTED, "quantize: group must be 0 or 64");
    if (group == 64 && cols % 64) return fail(COLI_EINVAL, "quantize: group 64 needs cols % 64 == 0");
    if (rows > 0 && (!d_w || !d_q || !d_s)) return fail(COLI_EINVAL, "quantize: NULL pointer");
    return launch_quantize(d_w, rows, cols, group, d_q, d_s, (hipStream_t)stream);
    COLI_GUARD_END
}

coli_status coli_quantize_expert(const coli_moe_shape* shape, const float* d_gate, const float* d_up,
                                 const float* d_down, void* d_blob, void* stream) {
    COLI_GUARD_BEGIN
    coli_status st = check_shape(shape);
    if (st) return st;
    if (!d_gate || !d_up || !d_down || !d_blob) return fail(COLI_EINVAL, "quantize_expert: NULL pointer");
    const int64_t H = shape->hidden, I = shape->inter;
    const int32_t wb = shape->wbits == 8 ? 8 : 4;
    const BlobLayout L = blob_layout(H, I, shape->group, wb);
    uint8_t* b = (uint8_t*)d_blob;
    hipStream_t s = (hipStream_t)stream;
    return launch_quantize_expert(d_gate, b + L.gate_q, (float*)(b + L.gate_s), d_up, b + L.up_q,
                                  (float*)(b + L.up_s), d_down, b + L.down_q, (float*)(b + L.down_s),
                                  H, I, shape->group, s, wb);
    COLI_GUARD_END
}

coli_status coli_convert_fp8_int4(const uint8_t* d_w8, const float* d_scale, int64_t rows,
                                  int64_t cols, int32_t group, uint8_t* d_q, float* d_s,
                                  void* stream) {
    COLI_GUARD_BEGIN
    if (rows < 0 || cols <= 0 || (cols & 1)) return fail(COLI_EINVAL, "convert_fp8: rows >= 0, cols even and > 0");
    if (group != 0 && group != 64) return fail(COLI_EUNSUPPORTED, "convert_fp8: group must be 0 or 64");
    if (group == 64 && cols % 64) return fail(COLI_EINVAL, "convert_fp8: group 64 needs cols % 64 == 0");
    if (rows > 0 && (!d_w8 || !d_scale || !d_q || !d_s)) return fail(COLI_EINVAL, "convert_fp8: NULL pointer");
    return launch_convert_fp8(d_w8, d_scale, rows, cols, group, d_q, d_s, (hipStream_t)stream);
    COLI_GUARD_END
}

coli_status coli_convert_fp8_expert(const coli_moe_shape* shape, const uint8_t* d_gate8,
                                    const float* d_gate_scale, const uint8_t* d_up8,
                                    const float* d_up_scale, const uint8_t* d_down8,
                                    const float* d_down_scale, void* d_blob, void* stream) {
    COLI_GUARD_BEGIN
    coli_status st = check_shape(shape);
    if (st) return st;
    if (!d_gate8 || !d_gate_scale || !d_up8 || !d_up_scale || !d_down8 || !d_down_scale || !d_blob)
        return fail(COLI_EINVAL, "convert_fp8_expert: NULL pointer");
    const int64_t H = shape->hidden, I = shape->inter;
    const int32_t wb = shape->wbits == 8 ? 8 : 4;
    const BlobLayout L = blob_layout(H, I, shape->group, wb);
    uint8_t* b = (uint8_t*)d_blob;
    hipStream_t s = (hipStream_t)stream;
    st = launch_convert_fp8_pair(d_gate8, d_gate_scale, b + L.gate_q, (float*)(b + L.gate_s),
                                 d_up8, d_up_scale, b + L.up_q, (float*)(b + L.up_s), I, H,
                                 shape->group, s, wb, true);
    if (st) return st;
    return launch_convert_fp8(d_down8, d_down_scale, H, I, shape->group, b + L.down_q,
                              (float*)(b + L.down_s), s, wb);
    COLI_GUARD_END
}

coli_status coli_moe_router_logits(const float* d_wr, const float* d_x, int32_t T, int32_t H,
                                   int32_t E, float* d_logits, void* stream) {
    COLI_GUARD_BEGIN
    if (T < 0 || H <= 0 || E <= 0) return fail(COLI_EINVAL, "router_logits: bad sizes");
    if (T > 0 && (!d_wr || !d_x || !d_logits)) return fail(COLI_EINVAL, "router_logits: NULL pointer");
    return launch_router_logits(d_wr, d_x, T, H, E, d_logits, (hipStream_t)stream);
    COLI_GUARD_END
}

static coli_status route_call(const float* d_logits, const float* d_bias, int32_t T, int32_t E,
                              int32_t k, float topp, int32_t* d_idx, float* d_w, void* stream) {
    if (T < 0 || E <= 0 || k <= 0 || k > E) return fail(COLI_EINVAL, "route: need T >= 0, 1 <= k <= E");
    if (E > 1024 || k > 32) return fail(COLI_EUNSUPPORTED, "route: E <= 1024 and k <= 32");
    if (!(topp >= 0.f && topp <= 1.f)) return fail(COLI_EINVAL, "route: topp must be in [0, 1]");
    if (T > 0 && (!d_logits || !d_idx || !d_w)) return fail(COLI_EINVAL, "route: NULL pointer");
    return launch_route(d_logits, d_bias, T, E, k, topp, d_idx, d_w, (hipStream_t)stream);
}

coli_status coli_moe_route(const float* d_logits, const float* d_bias, int32_t T, int32_t E,
                           int32_t k, int32_t* d_idx, float* d_w, void* stream) {
    COLI_GUARD_BEGIN
    return route_call(d_logits, d_bias, T, E, k, 0.f, d_idx, d_w, stream);
    COLI_GUARD_END
}

coli_status coli_moe_route_topp(const float* d_logits, const float* d_bias, int32_t T, int32_t E,
                                int32_t k, float topp, int32_t* d_idx, float* d_w, void* stream) {
    COLI_GUARD_BEGIN
    return route_call(d_logits, d_bias, T, E, k, topp, d_idx, d_w, stream);
    COLI_GUARD_END
}

coli_status coli_moe_union_workspace_size(int32_t T, int32_t k, int32_t E, size_t* bytes) {
    COLI_GUARD_BEGIN
    if (T < 0 || k <= 0 || E <= 0 || !bytes) return fail(COLI_EINVAL, "union_workspace_size: bad arguments");
    *bytes = union_ws_bytes(T, k, E);
    return COLI_OK;
    COLI_GUARD_END
}

coli_status coli_moe_union(const int32_t* d_idx, int32_t T, int32_t k, int32_t E, int32_t* d_counts,
                           int32_t* d_offsets, int32_t* d_perm, int32_t* d_unique,
                           int32_t* d_n_unique, void* d_ws, size_t ws_bytes, void* stream) {
    COLI_GUARD_BEGIN
    if (T < 0 || k <= 0 || E <= 0) return fail(COLI_EINVAL, "union: bad sizes");
    if (E > 1024) return fail(COLI_EUNSUPPORTED, "union: E <= 1024");
    if ((int64_t)T * k > (1 << 26)) return fail(COLI_EUNSUPPORTED, "union: T*k too large");
    if (!d_counts || !d_offsets || !d_unique || !d_n_unique || (T > 0 && (!d_idx || !d_perm)))
        return fail(COLI_EINVAL, "union: NULL pointer");
    if (ws_bytes < union_ws_bytes(T, k, E) || !d_ws) return fail(COLI_ENOMEM, "union: workspace too small");
    return launch_union(d_idx, T, k, E, d_counts, d_offsets, d_perm, d_unique, d_n_unique, d_ws,
                        (hipStream_t)stream);
    COLI_GUARD_END
}

coli_status coli_moe_workspace_size(const coli_moe_shape* shape, int32_t T, int32_t path, size_t* bytes) {
    COLI_GUARD_BEGIN
    coli_status st = check_shape(shape);
    if (st) return st;
    if (T < 0 || !bytes) return fail(COLI_EINVAL, "workspace_size: bad arguments");
    *bytes = ws_layout(shape, T, path).bytes;
    return COLI_OK;
    COLI_GUARD_END
}

coli_status coli_moe_expert_ffn(const coli_moe_shape* shape, const void* const* d_blob_table,
                                const float* d_x, int32_t T, const int32_t* d_offsets,
                                const int32_t* d_perm, const int32_t* d_unique,
                                const int32_t* d_n_unique, float* d_y_assign, int32_t path,
                                void* d_ws, size_t ws_bytes, void* stream) {
    COLI_GUARD_BEGIN
    coli_status st = check_shape(shape);
    if (st) return st;
    if (T < 0) return fail(COLI_EINVAL, "expert_ffn: T < 0");
    if (path < 0 || path > 2) return fail(COLI_EINVAL, "expert_ffn: path must be 0, 1 or 2");
    if (T == 0) return COLI_OK;
    if (!d_blob_table || !d_x || !d_offsets || !d_perm || !d_unique || !d_n_unique || !d_y_assign)
        return fail(COLI_EINVAL, "expert_ffn: NULL pointer");
    const WsLayout W = ws_layout(shape, T, path);
    if (!d_ws || ws_bytes < W.bytes) return fail(COLI_ENOMEM, "expert_ffn: workspace too small");
    return run_expert_ffn(shape, d_blob_table, d_x, T, d_offsets, d_perm, d_unique, d_n_unique,
                          d_y_assign, path, (uint8_t*)d_ws, W, (hipStream_t)stream);
    COLI_GUARD_END
}

coli_status coli_moe_layer_fwd(const coli_moe_shape* shape, const float* d_x, int32_t T,
                               const float* d_logits, const float* d_router_w, const float* d_bias,
                               const void* const* d_blob_table, const void* d_shared_blob,
                               struct coli_expert_cache* cache, int32_t layer, float* d_y,
                               int32_t* d_idx_out, float* d_w_out, int32_t path, void* d_ws,
                               size_t ws_bytes, void* stream) {
    COLI_GUARD_BEGIN
    coli_status st = check_shape(shape);
    if (st) return st;
    if (T < 0) return fail(COLI_EINVAL, "layer_fwd: T < 0");
    if (path < 0 || path > 2) return fail(COLI_EINVAL, "layer_fwd: path must be 0, 1 or 2");
    if ((d_logits == nullptr) == (d_router_w == nullptr))
        return fail(COLI_EINVAL, "layer_fwd: give exactly one of logits and router_w");
    if (shape->n_shared == 1 && !d_shared_blob) return fail(COLI_EINVAL, "layer_fwd: shared blob missing");
    if (!cache && !d_blob_table) return fail(COLI_EINVAL, "layer_fwd: blob table missing");
    if (T == 0) return COLI_OK;
    if (!d_x || !d_y) return fail(COLI_EINVAL, "layer_fwd: NULL pointer");
    const WsLayout W = ws_layout(shape, T, path);
    if (!d_ws || ws_bytes < W.bytes) return fail(COLI_ENOMEM, "layer_fwd: workspace too small");
    return run_layer(shape, d_x, T, d_logits, d_router_w, d_bias, d_blob_table,
                     shape->n_shared ? d_shared_blob : nullptr, cache, layer, d_y, d_idx_out,
                     d_w_out, path, (uint8_t*)d_ws, W, (hipStream_t)stream);
    COLI_GUARD_END
}

coli_status coli_moe_layer_fwd_noalloc(const coli_moe_shape* shape, const float* d_x, int32_t T,
                                       const float* d_logits, const float* d_router_w,
                                       const float* d_bias, const void* const* d_blob_table,
                                       const void* d_shared_blob, float* d_y, int32_t* d_idx_out,
                                       float* d_w_out, int32_t path, void* stream) {
    COLI_GUARD_BEGIN
    coli_status st = check_shape(shape);
    if (st) return st;
    if (T < 0) return fail(COLI_EINVAL, "layer_fwd_noalloc: T < 0");
    if (path < 0 || path > 2) return fail(COLI_EINVAL, "layer_fwd_noalloc: path must be 0, 1 or 2");
    if ((d_logits == nullptr) == (d_router_w == nullptr))
        return fail(COLI_EINVAL, "layer_fwd_noalloc: give exactly one of logits and router_w");
    if (shape->n_shared == 1 && !d_shared_blob) return fail(COLI_EINVAL, "layer_fwd_noalloc: shared blob missing");
    if (!d_blob_table) return fail(COLI_EINVAL, "layer_fwd_noalloc: blob table missing");
    if (T == 0) return COLI_OK;
    if (!d_x || !d_y) return fail(COLI_EINVAL, "layer_fwd_noalloc: NULL pointer");
    const WsLayout W = ws_layout(shape, T, path);
    if (W.bytes > kScratchBytes)
        return fail(COLI_ENOMEM, "layer_fwd_noalloc: this call needs " + std::to_string(W.bytes) +
                                 " bytes of scratch; the static scratch holds " +
                                 std::to_string(kScratchBytes) +
                                 " (use coli_moe_layer_fwd with a workspace, or fewer tokens)");
    uint8_t* ws = nullptr;
    st = scratch_on_current_device(&ws);
    if (st) return st;
    return run_layer(shape, d_x, T, d_logits, d_router_w, d_bias, d_blob_table,
                     shape->n_shared ? d_shared_blob : nullptr, nullptr, 0, d_y, d_idx_out,
                     d_w_out, path, ws, W, (hipStream_t)stream);
    COLI_GUARD_END
}

coli_status coli_profile_rerun(const coli_moe_shape* shape, int32_t T,
                              const void* const* d_blob_table, const void* d_shared_blob,
                              int32_t which, void* d_ws, size_t ws_bytes, void* stream) {
    COLI_GUARD_BEGIN
    coli_status st = check_shape(shape);
    if (st) return st;
    if (T <= 0 || T > kSmallT) return fail(COLI_EINVAL, "profile_rerun: T must be in [1, 16]");
    if (which != 0 && which != 1) return fail(COLI_EINVAL, "profile_rerun: which must be 0 or 1");
    if (!d_blob_table) return fail(COLI_EINVAL, "profile_rerun: blob table missing");
    if (shape->n_shared == 1 && !d_shared_blob) return fail(COLI_EINVAL, "profile_rerun: shared blob missing");
    const WsLayout W = ws_layout(shape, T, COLI_PATH_GEMV);
    if (!d_ws || ws_bytes < W.bytes) return fail(COLI_ENOMEM, "profile_rerun: workspace too small");
    return run_rerun(shape, T, d_blob_table, shape->n_shared ? d_shared_blob : nullptr, which,
                     (uint8_t*)d_ws, W, (hipStream_t)stream);
    COLI_GUARD_END
}

coli_status coli_moe_lookahead(const coli_moe_shape* shape, const float* d_x, int32_t T,
                               const float* d_logits, const float* d_router_w, const float* d_bias,
                               struct coli_expert_cache* cache, int32_t layer, int32_t* h_started,
                               void* d_ws, size_t ws_bytes, void* stream) {
    COLI_GUARD_BEGIN
    coli_status st = check_shape(shape);
    if (st) return st;
    if (T < 0 || !cache) return fail(COLI_EINVAL, "lookahead: T < 0 or no cache");
    if ((d_logits == nullptr) == (d_router_w == nullptr))
        return fail(COLI_EINVAL, "lookahead: give exactly one of logits and router_w");
    if (h_started) *h_started = 0;
    if (T == 0) return COLI_OK;
    if (d_router_w && !d_x) return fail(COLI_EINVAL, "lookahead: NULL x");
    const WsLayout W = ws_layout(shape, T, COLI_PATH_AUTO);
    if (!d_ws || ws_bytes < W.bytes) return fail(COLI_ENOMEM, "lookahead: workspace too small");
    return run_lookahead(shape, d_x, T, d_logits, d_router_w, d_bias, cache, layer, h_started,
                         (uint8_t*)d_ws, W, (hipStream_t)stream);
    COLI_GUARD_END
}

}  // extern "C"
