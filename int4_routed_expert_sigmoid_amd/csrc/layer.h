// Internal: workspace layout and the launch sequences behind the C ABI.
#pragma once

#include "common.h"

namespace coli {

struct WsLayout {
    size_t logits, idx, w, counts, offsets, perm, unique, n_unique, n_items, union_ws, items,
        rows_tok, rows_out, xplanes, xscale, hplanes, hscale, y_rows, phase, tiles, n_tiles, gv_items,
        n_gv, xb, sx, hb, sh,
        codes, scores, bytes;
    size_t max_tiles;
};

coli_status check_shape(const coli_moe_shape* s);
WsLayout ws_layout(const coli_moe_shape* s, int32_t T, int32_t path);

coli_status run_expert_ffn(const coli_moe_shape* shape, const void* const* table, const float* x,
                           int32_t T, const int32_t* offsets, const int32_t* perm,
                           const int32_t* unique, const int32_t* n_unique, float* y_assign,
                           int32_t path, uint8_t* ws, const WsLayout& W, hipStream_t stream);

coli_status run_layer(const coli_moe_shape* shape, const float* x, int32_t T, const float* logits,
                      const float* router_w, const float* bias, const void* const* table,
                      const void* shared_blob, struct coli_expert_cache* cache, int32_t layer,
                      float* y, int32_t* idx_out, float* w_out, int32_t path, uint8_t* ws,
                      const WsLayout& W, hipStream_t stream);

// One GEMV pass (which: 0 gate/up, 1 down) of the last uncached GEMV-path
// layer call on ws, enqueued again (measurement).
coli_status run_rerun(const coli_moe_shape* shape, int32_t T, const void* const* table,
                      const void* shared_blob, int32_t which, uint8_t* ws, const WsLayout& W,
                      hipStream_t stream);

// Expert-cache hooks used by run_layer (cache.hip).
coli_status cache_layer_table(struct coli_expert_cache* cache, int32_t layer, int32_t n_experts,
                              const void* const** table);
coli_status cache_place(struct coli_expert_cache* cache, int32_t layer, const int32_t* d_idx,
                        int32_t n, uint8_t* d_phase, int32_t* n_miss, hipStream_t stream);
coli_status cache_prefetch_routed(struct coli_expert_cache* cache, int32_t layer,
                                  const int32_t* d_idx, int32_t n, int32_t* started,
                                  hipStream_t stream);

coli_status run_lookahead(const coli_moe_shape* shape, const float* x, int32_t T,
                          const float* logits, const float* router_w, const float* bias,
                          struct coli_expert_cache* cache, int32_t layer, int32_t* started,
                          uint8_t* ws, const WsLayout& W, hipStream_t stream);

}  // namespace coli
