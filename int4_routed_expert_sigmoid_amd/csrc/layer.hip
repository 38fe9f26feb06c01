// Launch sequences of coli_moe_expert_ffn and coli_moe_layer_fwd.
//
// Practical guide section 二: per token and layer, route -> union -> place ->
// execute (-> learn). Everything below is enqueued on the caller's stream;
// nothing waits on the host except the cached layer, which must read the
// routing back to decide placement.
#include <algorithm>
#include <vector>

#include "gemm.h"
#include "gemv.h"
#include "layer.h"

namespace coli {

template <typename T>
static T* at(uint8_t* ws, size_t off) { return reinterpret_cast<T*>(ws + off); }

// Decide the FFN path: the GEMV family for small batches, the bf16 MFMA
// grouped GEMM for large ones (auto), or the caller's choice. *split: with
// the MFMA path chosen automatically, experts with at most kGemvMaxTokens
// tokens run on the GEMV family (the batch union reads each of them once
// either way; for so few tokens a dense tile would be mostly padding).
static coli_status pick_mfma(const coli_moe_shape* s, int32_t T, int32_t path, bool* mfma,
                             bool* split = nullptr) {
    // the MFMA path dequantises int4 weights only; int8 experts always take the GEMV family
    const bool int8 = s->wbits == 8;
    const bool shape_ok = s->hidden % 64 == 0 && s->inter % 64 == 0 && !int8;
    if (split) *split = false;
    if (path == COLI_PATH_MFMA) {
        if (int8) return fail(COLI_EUNSUPPORTED, "mfma path: int4 weights only");
        if (!shape_ok) return fail(COLI_EUNSUPPORTED, "mfma path: hidden and inter must be multiples of 64");
        *mfma = true;
    } else if (path == COLI_PATH_GEMV) {
        *mfma = false;
    } else {
        *mfma = shape_ok && T > kSmallT;
        if (split) *split = *mfma;
    }
    return COLI_OK;
}

static coli_status run_ffn(const coli_moe_shape* s, bool mfma, const float* x, int32_t T,
                           int32_t max_items, float* y_rows, uint8_t* ws, const WsLayout& W,
                           bool x_encoded, hipStream_t stream, const FusedRoute* fused = nullptr,
                           int passes = kPassBoth, bool split = false) {
    const int32_t H = s->hidden, I = s->inter;
    if (mfma) {
        GemmArgs g;
        g.items = at<WorkItem>(ws, W.items);
        g.n_items = at<int32_t>(ws, W.n_items);
        g.rows_tok = at<int32_t>(ws, W.rows_tok);
        g.rows_out = at<int32_t>(ws, W.rows_out);
        g.tiles = at<int2>(ws, W.tiles);
        g.n_tiles = at<int32_t>(ws, W.n_tiles);
        g.xb = at<uint16_t>(ws, W.xb);
        g.sx = at<float>(ws, W.sx);
        g.hb = at<uint16_t>(ws, W.hb);
        g.sh = at<float>(ws, W.sh);
        g.y_rows = y_rows;
        g.L = blob_layout(H, I, s->group);
        g.H = H; g.I = I; g.group = s->group;
        g.gv_max = split ? kGemvMaxTokens : 0;
        g.gv_items = at<WorkItem>(ws, W.gv_items);
        g.n_gv = at<int32_t>(ws, W.n_gv);
        const int32_t rows = (int32_t)((int64_t)T * s->top_k + T);
        const int32_t max_tiles = (int32_t)gemm_tiles_max(rows, max_items);
        coli_status st = launch_mfma_ffn(g, x, T, max_tiles, stream);
        if (st || !split) return st;
        // the experts with few tokens: GEMV family over the compacted list,
        // with the digit planes of just the x rows it reads
        const int32_t* rows_tok = at<int32_t>(ws, W.rows_tok);
        const int32_t* rows_out = at<int32_t>(ws, W.rows_out);
        st = launch_encode_items(g.gv_items, g.n_gv, max_items, kGemvMaxTokens, rows_tok, x, H,
                                 at<uint32_t>(ws, W.xplanes), at<float>(ws, W.xscale), stream);
        if (st) return st;
        FusedRoute none{};
        return launch_gemv_ffn(g.gv_items, g.n_gv, max_items, kGemvMaxTokens, rows_tok, rows_out,
                               at<uint32_t>(ws, W.xplanes), at<float>(ws, W.xscale),
                               at<uint32_t>(ws, W.hplanes), at<float>(ws, W.hscale), y_rows, H, I,
                               s->group, s->wbits, none, stream, kPassBoth);
    }
    if (!x_encoded) {
        coli_status st = launch_encode(x, T, H, at<uint32_t>(ws, W.xplanes), at<float>(ws, W.xscale), stream);
        if (st) return st;
    }
    FusedRoute none{};
    return launch_gemv_ffn(at<WorkItem>(ws, W.items), at<int32_t>(ws, W.n_items), max_items, T,
                           at<int32_t>(ws, W.rows_tok), at<int32_t>(ws, W.rows_out),
                           at<uint32_t>(ws, W.xplanes), at<float>(ws, W.xscale),
                           at<uint32_t>(ws, W.hplanes), at<float>(ws, W.hscale), y_rows, H, I,
                           s->group, s->wbits, fused ? *fused : none, stream, passes);
}

// One token on the GEMV path without a cache: the routing is folded into the
// gate/up pass.
static bool folds_routing(const coli_moe_shape* s, int32_t T, bool cached, bool mfma) {
    return T == 1 && !cached && !mfma && s->n_routed <= kFusedMaxExperts;
}

static FusedRoute fused_route(const coli_moe_shape* s, const void* const* table,
                              const void* shared_blob, int32_t* idx, float* w, uint8_t* ws,
                              const WsLayout& W) {
    FusedRoute fr{};
    fr.codes = at<uint64_t>(ws, W.codes);
    fr.scores = at<float>(ws, W.scores);
    fr.table = table;
    fr.shared = shared_blob;
    fr.E = s->n_routed;
    fr.k = s->top_k;
    fr.topp = s->topp;
    fr.idx = idx;
    fr.w = w;
    fr.rows_tok = at<int32_t>(ws, W.rows_tok);
    fr.rows_out = at<int32_t>(ws, W.rows_out);
    fr.items = at<WorkItem>(ws, W.items);
    fr.n_items = at<int32_t>(ws, W.n_items);
    return fr;
}

coli_status run_expert_ffn(const coli_moe_shape* s, const void* const* table, const float* x,
                           int32_t T, const int32_t* offsets, const int32_t* perm,
                           const int32_t* unique, const int32_t* n_unique, float* y_assign,
                           int32_t path, uint8_t* ws, const WsLayout& W, hipStream_t stream) {
    const int32_t E = s->n_routed, k = s->top_k;
    bool mfma = false, split = false;
    coli_status st = pick_mfma(s, T, path, &mfma, &split);
    if (st) return st;
    st = launch_plan(offsets, perm, unique, n_unique, table, nullptr, T, k, E, nullptr, 0,
                     at<WorkItem>(ws, W.items), at<int32_t>(ws, W.n_items),
                     at<int32_t>(ws, W.rows_tok), at<int32_t>(ws, W.rows_out), stream);
    if (st) return st;
    const int32_t max_items = (int32_t)std::min<int64_t>(E, (int64_t)T * k);
    return run_ffn(s, mfma, x, T, max_items, y_assign, ws, W, false, stream, nullptr, kPassBoth,
                   split);
}

coli_status run_layer(const coli_moe_shape* s, const float* x, int32_t T, const float* logits,
                      const float* router_w, const float* bias, const void* const* table,
                      const void* shared_blob, struct coli_expert_cache* cache, int32_t layer,
                      float* y, int32_t* idx_out, float* w_out, int32_t path, uint8_t* ws,
                      const WsLayout& W, hipStream_t stream) {
    const int32_t H = s->hidden, E = s->n_routed, k = s->top_k;
    if (cache) {
        coli_status cs = cache_layer_table(cache, layer, E, &table);
        if (cs) return cs;
    }
    // with a cache the work items are formed after placement (table unused here)
    const void* const* route_table = cache ? nullptr : table;
    bool mfma = false, split = false;
    coli_status st = pick_mfma(s, T, path, &mfma, &split);
    if (st) return st;
    int32_t* idx = idx_out ? idx_out : at<int32_t>(ws, W.idx);
    float* w = w_out ? w_out : at<float>(ws, W.w);
    bool encoded = false;
    // one token on the GEMV path: the gate/up pass routes (no separate plan pass)
    const bool fold = folds_routing(s, T, cache != nullptr, mfma);
    const FusedRoute fr = fold ? fused_route(s, table, shared_blob, idx, w, ws, W) : FusedRoute{};
    if (T <= kSmallT) {
        // router: logits + activation encoding, then route / union / work list
        SmallRouterArgs ra;
        ra.x = x; ra.router_w = router_w; ra.logits_in = logits; ra.bias = bias;
        ra.logits_out = at<float>(ws, W.logits);
        ra.idx = idx; ra.w = w;
        ra.counts = at<int32_t>(ws, W.counts); ra.offsets = at<int32_t>(ws, W.offsets);
        ra.perm = at<int32_t>(ws, W.perm); ra.unique = at<int32_t>(ws, W.unique);
        ra.n_unique = at<int32_t>(ws, W.n_unique);
        ra.items = at<WorkItem>(ws, W.items); ra.n_items = at<int32_t>(ws, W.n_items);
        ra.rows_tok = at<int32_t>(ws, W.rows_tok); ra.rows_out = at<int32_t>(ws, W.rows_out);
        ra.xplanes = at<uint32_t>(ws, W.xplanes); ra.xscale = at<float>(ws, W.xscale);
        ra.table = route_table; ra.shared_blob = shared_blob;
        ra.phase_mask = nullptr; ra.phase = 0;
        ra.T = T; ra.E = E; ra.k = k; ra.H = H;
        ra.topp = s->topp;
        ra.codes = fold ? at<uint64_t>(ws, W.codes) : nullptr;
        ra.scores = fold ? at<float>(ws, W.scores) : nullptr;
        ra.split = !mfma ? 1 : 0;
        st = launch_router_small(ra, stream);
        if (st) return st;
        encoded = true;
    } else {
        const float* lg = logits;
        if (!lg) {
            st = launch_router_logits(router_w, x, T, H, E, at<float>(ws, W.logits), stream);
            if (st) return st;
            lg = at<float>(ws, W.logits);
        }
        st = launch_route(lg, bias, T, E, k, s->topp, idx, w, stream);
        if (st) return st;
        st = launch_union(idx, T, k, E, at<int32_t>(ws, W.counts), at<int32_t>(ws, W.offsets),
                          at<int32_t>(ws, W.perm), at<int32_t>(ws, W.unique),
                          at<int32_t>(ws, W.n_unique), ws + W.union_ws, stream);
        if (st) return st;
        if (!cache) {
            st = launch_plan(at<int32_t>(ws, W.offsets), at<int32_t>(ws, W.perm),
                             at<int32_t>(ws, W.unique), at<int32_t>(ws, W.n_unique), table,
                             shared_blob, T, k, E, nullptr, 0, at<WorkItem>(ws, W.items),
                             at<int32_t>(ws, W.n_items), at<int32_t>(ws, W.rows_tok),
                             at<int32_t>(ws, W.rows_out), stream);
            if (st) return st;
        }
    }
    // small batches on the GEMV path split their experts into items of at most
    // kItemTokens tokens (one token: every item has one)
    const bool split_items = T > 1 && T <= kSmallT && !cache && !mfma;
    const int32_t max_items = split_items
        ? (int32_t)split_items_bound(E, T, k, shared_blob != nullptr)
        : (int32_t)std::min<int64_t>(E, (int64_t)T * k) + (shared_blob ? 1 : 0);
    if (!cache) {
        st = run_ffn(s, mfma, x, T, max_items, at<float>(ws, W.y_rows), ws, W, encoded, stream,
                     fold ? &fr : nullptr, kPassBoth, split);
        if (st) return st;
    } else {
        // place: read the routing back, make the experts resident (misses are
        // copied on the cache's copy stream), upload each expert's phase
        uint8_t* d_phase = at<uint8_t>(ws, W.phase);
        int32_t n_miss = 0;
        st = cache_place(cache, layer, idx, T * k, d_phase, &n_miss, stream);
        if (st) return st;
        // execute the experts that were resident (and the shared one) while the
        // misses copy, then wait for the copies and execute the misses
        for (int phase = 0; phase < (n_miss > 0 ? 2 : 1); ++phase) {
            if (phase == 1) {
                st = coli_expert_cache_wait(cache, layer, (void*)stream);
                if (st) return st;
            }
            st = launch_plan(at<int32_t>(ws, W.offsets), at<int32_t>(ws, W.perm),
                             at<int32_t>(ws, W.unique), at<int32_t>(ws, W.n_unique), table,
                             phase == 0 ? shared_blob : nullptr, T, k, E, d_phase, phase,
                             at<WorkItem>(ws, W.items), at<int32_t>(ws, W.n_items),
                             at<int32_t>(ws, W.rows_tok), at<int32_t>(ws, W.rows_out), stream);
            if (st) return st;
            st = run_ffn(s, mfma, x, T, max_items, at<float>(ws, W.y_rows), ws, W,
                         encoded || phase == 1, stream, nullptr, kPassBoth, split);
            if (st) return st;
        }
        st = coli_expert_cache_release(cache, layer, (void*)stream);
        if (st) return st;
    }
    // with the adaptive top-p some slots are dropped (index -1, no output row)
    const bool adaptive = s->topp > 0.f && s->topp < 1.f;
    return launch_combine(at<float>(ws, W.y_rows), w, adaptive ? idx : nullptr, T, k, H,
                          shared_blob ? 1 : 0, s->routed_scale, y, stream);
}

coli_status run_rerun(const coli_moe_shape* s, int32_t T, const void* const* table,
                      const void* shared_blob, int32_t which, uint8_t* ws, const WsLayout& W,
                      hipStream_t stream) {
    bool mfma = false;
    coli_status st = pick_mfma(s, T, COLI_PATH_GEMV, &mfma);
    if (st) return st;
    const int32_t E = s->n_routed, k = s->top_k;
    // the work list the layer call left: split items for small batches
    const int32_t max_items = T > 1 && T <= kSmallT
        ? (int32_t)split_items_bound(E, T, k, shared_blob != nullptr)
        : (int32_t)std::min<int64_t>(E, (int64_t)T * k) + (shared_blob ? 1 : 0);
    // the routing the gate/up pass republishes goes to the workspace's own copy
    const bool fold = folds_routing(s, T, false, false);
    const FusedRoute fr = fold ? fused_route(s, table, shared_blob, at<int32_t>(ws, W.idx),
                                             at<float>(ws, W.w), ws, W)
                               : FusedRoute{};
    return run_ffn(s, false, nullptr, T, max_items, at<float>(ws, W.y_rows), ws, W, true, stream,
                   fold ? &fr : nullptr, which == 0 ? kPassGateUp : kPassDown);
}

coli_status run_lookahead(const coli_moe_shape* s, const float* x, int32_t T, const float* logits,
                          const float* router_w, const float* bias, coli_expert_cache* cache,
                          int32_t layer, int32_t* started, uint8_t* ws, const WsLayout& W,
                          hipStream_t stream) {
    const int32_t H = s->hidden, E = s->n_routed, k = s->top_k;
    const void* const* table = nullptr;
    coli_status cs = cache_layer_table(cache, layer, E, &table);   // checks layer and E
    if (cs) return cs;
    const float* lg = logits;
    if (!lg) {
        coli_status st = launch_router_logits(router_w, x, T, H, E, at<float>(ws, W.logits), stream);
        if (st) return st;
        lg = at<float>(ws, W.logits);
    }
    coli_status st = launch_route(lg, bias, T, E, k, s->topp, at<int32_t>(ws, W.idx),
                                  at<float>(ws, W.w), stream);
    if (st) return st;
    return cache_prefetch_routed(cache, layer, at<int32_t>(ws, W.idx), T * k, started, stream);
}

}  // namespace coli
