/*
 * libcoli_moe: one int4 routed-expert MoE layer with a sigmoid router, for
 * MI355X (gfx950). C ABI: plain pointers and sizes, no C++ or torch types.
 *
 * The layer, per token (practical guide "colibrì 實戰指南：以純 C 引擎在消費級
 * 硬體上串流運行 744B MoE 模型", section 二: route -> union -> place ->
 * overlapped execute -> learn):
 *   1. route: sigmoid scores of the router logits, a per-expert bias added for
 *      selection only, the top-k experts by biased key, weights = unbiased
 *      scores normalised over the k selected (lbrq.cn article "github一周涨
 *      11k⭐️！25GB 内存跑 744B GLM-5.2 模型！", section 三 item 1 and section 四
 *      item 3; config.json values sigmoid / norm_topk_prob quoted by the
 *      int8-MTP page "解密GLM-5.2-colibri-int4-with-int8-mtp…").
 *   2. union: the T*k (token, slot) assignments grouped by expert, so each
 *      unique expert's weights are read once for all of its tokens (lbrq.cn
 *      article section 三 item 4; practical guide section 二).
 *   3. place: an HBM cache of expert blobs in front of pinned host memory
 *      (practical guide section 二: per-layer LRU, one read per expert,
 *      misses loaded while resident experts compute).
 *   4. execute: each selected expert and the shared expert is an int4 SwiGLU
 *      FFN, y_e = down(silu(gate x) * (up x)); the layer output is
 *      y = shared(x) + routed_scale * sum_j w_j y_{e_j}, summed in slot order.
 *
 * Quantised format (model card "jlnsrk/GLM-5.2-colibri-int4": U8 packed int4
 * nibbles plus F32 scales, rounded with np.rint / lrintf; gs64 groups from
 * the practical guide section 三): scale = max|w|/7 per row (group 0) or per
 * 64 consecutive inputs of a row (group 64); q = rint(w/scale) in float,
 * half-to-even, clamped to [-8, 7]; two's-complement nibbles, column 2i in
 * bits 0-3 and 2i+1 in bits 4-7 of byte i; rows are row-major.
 *
 * Expert blob: one contiguous device buffer per expert holding, in order,
 * the rows of gate_q and up_q (each [I][H/2] u8) interleaved in blocks of 16
 * rows (rows 16b..16b+15 of gate, then the same rows of up, for b = 0, 1, ...;
 * so the gate rows start at the gate_q offset and the up rows 16 rows later,
 * each with a block stride of 32 rows), then down_q [H][I/2] (u8), gate_s,
 * up_s ([I] or [I][H/64] f32) and down_s ([H] or [H][I/64] f32); every part
 * starts on a 256-byte boundary (coli_expert_blob_layout gives the offsets).
 * A workgroup that reads rows of both matrices reads one contiguous stretch,
 * and a miss of the expert cache is one copy.
 *
 * int8 experts (shape->wbits 8; the MTP head must be int8 per the int8-MTP
 * page and the practical guide's section 二, and the pages give no int8
 * formula): scale = max|w|/127 per row or 64-group, q = rint(w/scale)
 * half-to-even clamped to [-128, 127]. The blob has the same parts with rows of
 * H (or I) bytes: for every 32-element block, 16 bytes holding the high
 * nibbles h = q >> 4, then 16 bytes holding l = (q & 15) - 8, both as signed
 * nibbles in the int4 packing order, so that q = 16 h + l + 8. int8 layers run
 * on the GEMV family only (COLI_PATH_MFMA returns COLI_EUNSUPPORTED).
 *
 * Conventions for every call:
 *  - d_* pointers are device memory, h_* pointers host memory. The caller owns
 *    all of them; the library keeps none after a call returns (the expert
 *    cache handle's pools and arena, and the buffers of the testing read log,
 *    coli_debug_read_log, aside).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work on it and return, unless stated otherwise.
 *  - Return value: COLI_OK, or a negative code with a message readable via
 *    coli_last_error() (thread-local, valid until the next call on the same
 *    thread). Argument errors are found before anything is enqueued. Faults
 *    inside kernels surface at the caller's next synchronisation, as for any
 *    HIP stream work.
 *  - Floating-point inputs must be finite.
 */
#ifndef COLI_MOE_H
#define COLI_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define COLI_API __attribute__((visibility("default")))
#else
#define COLI_API
#endif

typedef int32_t coli_status;
#define COLI_OK 0
#define COLI_EINVAL (-1)        /* null pointer, bad size or shape */
#define COLI_EUNSUPPORTED (-2)  /* valid but outside the supported ranges */
#define COLI_EHIP (-3)          /* a HIP call failed; message has hipGetErrorString */
#define COLI_ENOMEM (-4)        /* workspace too small or host allocation failed */
#define COLI_EBUSY (-5)         /* every cache slot of the layer is pinned by this call */

COLI_API const char* coli_last_error(void);
COLI_API const char* coli_version(void);

/* Layer shape. Supported: hidden <= 16384 and inter <= 4096, positive multiples of 32 (and of
 * 64 when group == 64); 1 <= n_routed <= 1024; n_shared 0 or 1;
 * 1 <= top_k <= min(32, n_routed); group 0 or 64; routed_scale finite; topp in [0, 1];
 * wbits 0, 4 or 8. */
typedef struct coli_moe_shape {
    int32_t hidden;       /* H: model width, input and output of the layer */
    int32_t inter;        /* I: intermediate width of one expert */
    int32_t n_routed;     /* E: routed experts */
    int32_t n_shared;     /* 0 or 1 shared expert, weight 1, always applied */
    int32_t top_k;        /* k: experts per token */
    int32_t group;        /* 0: one scale per row; 64: one scale per 64 inputs */
    float routed_scale;   /* multiplies the routed sum at the combine (1.0 = none) */
    float topp;           /* adaptive expert top-p, as coli_moe_route_topp: 0 (or 1) keeps
                             all top_k; in (0, 1) a token may use fewer experts (lossy) */
    int32_t wbits;        /* expert weight codec: 4 (or 0) int4, 8 int8 (GEMV path only) */
} coli_moe_shape;

/* Offsets (bytes) of gate_q, up_q, down_q, gate_s, up_s, down_s inside one
 * expert blob, and the blob size. Row r of gate is at gate_q + (32 (r / 16) +
 * r % 16) * row bytes, row r of up at up_q + the same (up_q = gate_q + 16 rows).
 * Host-only arithmetic. */
COLI_API coli_status coli_expert_blob_layout(const coli_moe_shape* shape, size_t off[6], size_t* blob_bytes);

/* Quantise d_w [rows][cols] (f32) to d_q [rows][cols/2] (u8) and d_s ([rows]
 * or [rows][cols/64] f32) by the rule above. Bit-identical to the CPU
 * reference for finite input. cols even (multiple of 64 for group 64). */
COLI_API coli_status coli_quantize_int4(const float* d_w, int64_t rows, int64_t cols, int32_t group,
                               uint8_t* d_q, float* d_s, void* stream);

/* Quantise one expert's three f32 matrices (gate/up [I][H], down [H][I]) into
 * the blob d_blob (coli_expert_blob_layout bytes). */
COLI_API coli_status coli_quantize_expert(const coli_moe_shape* shape, const float* d_gate,
                                 const float* d_up, const float* d_down, void* d_blob,
                                 void* stream);

/* FP8 -> f32 -> int4 converter (model card "jlnsrk/GLM-5.2-colibri-int4",
 * conversion note: the container was made from the FP8 checkpoint, e4m3 with
 * one scale per 128 x 128 block, via f32, rounding as np.rint). d_w8
 * [rows][cols] holds OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits, subnormals at exponent 0, no infinity; the NaN codes 0x7F and
 * 0xFF must not occur); d_scale is f32 [ceil(rows/128)][ceil(cols/128)]
 * row-major. Each weight is w = e4m3 value * scale of its block, one f32
 * rounding, then quantised exactly as coli_quantize_int4 does (bit-identical
 * to the CPU reference). Same size rules and outputs as coli_quantize_int4. */
COLI_API coli_status coli_convert_fp8_int4(const uint8_t* d_w8, const float* d_scale, int64_t rows,
                                  int64_t cols, int32_t group, uint8_t* d_q, float* d_s,
                                  void* stream);

/* One expert from its three FP8 matrices (gate/up [I][H], down [H][I], each
 * with its block scales) into the blob d_blob, like coli_quantize_expert. */
COLI_API coli_status coli_convert_fp8_expert(const coli_moe_shape* shape, const uint8_t* d_gate8,
                                    const float* d_gate_scale, const uint8_t* d_up8,
                                    const float* d_up_scale, const uint8_t* d_down8,
                                    const float* d_down_scale, void* d_blob, void* stream);

/* Router logits d_logits [T][E] = d_x [T][H] . d_wr [E][H]^T: f32 inputs,
 * products and sum in double, one rounding to f32 (the router stays F32 in
 * the container, model card file table). */
COLI_API coli_status coli_moe_router_logits(const float* d_wr, const float* d_x, int32_t T, int32_t H,
                                   int32_t E, float* d_logits, void* stream);

/* Sigmoid top-k routing of T tokens over E experts (E <= 1024, k <= 32).
 * score = sigmoid(logit) computed in double and rounded once to f32;
 * key = score + bias (f32; d_bias NULL means zero); the k largest keys in
 * descending order, equal keys to the lower expert index, into d_idx [T][k];
 * d_w [T][k] = score / (sum of the k selected scores, in slot order, double),
 * rounded to f32 (1/k if that sum is 0). */
COLI_API coli_status coli_moe_route(const float* d_logits, const float* d_bias, int32_t T, int32_t E,
                           int32_t k, int32_t* d_idx, float* d_w, void* stream);

/* coli_moe_route with an adaptive expert top-p (practical guide section 三,
 * where 0.7 is the setting recommended for disk-bound machines, and the
 * section 五 tuning table: an adaptive expert top-p that reads 30-40% fewer
 * expert bytes; lossy). The pages give no formula; this call takes the k
 * experts selected as above, in slot (key) order, and keeps the shortest
 * prefix whose share of the k selected scores reaches topp: slot j is kept iff
 * j == 0 or (s_0 + ... + s_{j-1}) / (s_0 + ... + s_{k-1}) < topp, sums in
 * double in slot order (j / k instead when all k scores are 0). The kept
 * weights are score / (sum of the kept scores, slot order, double), rounded to
 * f32 (1/kept if that sum is 0); dropped slots get d_idx -1 and d_w 0, at the
 * end of each row. topp 0 or 1 is coli_moe_route; outside [0, 1] (or NaN) is
 * COLI_EINVAL. */
COLI_API coli_status coli_moe_route_topp(const float* d_logits, const float* d_bias, int32_t T,
                                int32_t E, int32_t k, float topp, int32_t* d_idx, float* d_w,
                                void* stream);

/* Workspace bytes coli_moe_union needs for T tokens, k slots, E experts. */
COLI_API coli_status coli_moe_union_workspace_size(int32_t T, int32_t k, int32_t E, size_t* bytes);

/* Batch union of the T*k assignments a = t*k + j of d_idx [T][k]:
 * d_counts [E]; d_offsets [E+1] (exclusive prefix sum, offsets[E] = T*k);
 * d_perm [T*k]: assignments grouped by expert, ascending within a group;
 * d_unique [E]: the experts with count > 0, ascending, first *d_n_unique
 * entries valid. Deterministic (no atomics decide any order). Entries outside
 * [0, E) belong to no expert: they are left out of counts and perm, so
 * offsets[E] is then the number of valid entries. */
COLI_API coli_status coli_moe_union(const int32_t* d_idx, int32_t T, int32_t k, int32_t E,
                           int32_t* d_counts, int32_t* d_offsets, int32_t* d_perm,
                           int32_t* d_unique, int32_t* d_n_unique, void* d_ws, size_t ws_bytes,
                           void* stream);

#define COLI_PATH_AUTO 0   /* GEMV family for small per-expert counts, MFMA otherwise */
#define COLI_PATH_GEMV 1   /* int4 dequant GEMV family (f32-accurate) */
#define COLI_PATH_MFMA 2   /* bf16 MFMA grouped GEMM on dequantised tiles */

/* Workspace bytes for coli_moe_expert_ffn / coli_moe_layer_fwd with T tokens.
 * The workspace is device memory owned by the caller. It needs no
 * initialisation: every call writes each region it reads before reading it.
 * A workspace serves one call at a time: calls that share one must be ordered
 * on a stream. */
COLI_API coli_status coli_moe_workspace_size(const coli_moe_shape* shape, int32_t T, int32_t path,
                                    size_t* bytes);

/* Unweighted expert outputs for a union: for every unique expert e (first
 * *d_n_unique entries of d_unique) and every assignment a in d_perm
 * [d_offsets[e], d_offsets[e+1]), d_y_assign [a][H] = FFN_e(d_x [a / k]).
 * Rows of assignments of no listed expert are left untouched.
 * d_blob_table: device array [E] of device pointers to expert blobs. */
COLI_API coli_status coli_moe_expert_ffn(const coli_moe_shape* shape, const void* const* d_blob_table,
                                const float* d_x, int32_t T, const int32_t* d_offsets,
                                const int32_t* d_perm, const int32_t* d_unique,
                                const int32_t* d_n_unique, float* d_y_assign, int32_t path,
                                void* d_ws, size_t ws_bytes, void* stream);

struct coli_expert_cache;

/* One whole layer for T tokens: route, union, expert FFNs (routed + shared),
 * combine. Exactly one of d_logits [T][E] and d_router_w [E][H] is given.
 * d_bias [E] may be NULL. d_shared_blob is required iff shape->n_shared == 1.
 * Without a cache, d_blob_table [E] (device) gives the routed blobs. With a
 * cache, d_blob_table is ignored: the call copies the routing to the host
 * (one blocking 4*T*k-byte read), makes the selected experts of `layer`
 * resident, runs the resident ones while the misses are copied, then the
 * misses. d_idx_out [T][k] and d_w_out [T][k] (nullable) receive the routing.
 * With shape->topp in (0, 1) the routing is coli_moe_route_topp's: dropped
 * slots (index -1) are left out of the union and add nothing at the combine.
 * d_y [T][H] f32. */
COLI_API coli_status coli_moe_layer_fwd(const coli_moe_shape* shape, const float* d_x, int32_t T,
                               const float* d_logits, const float* d_router_w,
                               const float* d_bias, const void* const* d_blob_table,
                               const void* d_shared_blob, struct coli_expert_cache* cache,
                               int32_t layer, float* d_y, int32_t* d_idx_out, float* d_w_out,
                               int32_t path, void* d_ws, size_t ws_bytes, void* stream);

/* coli_moe_layer_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same launch sequence and results, with resident experts
 * only (no cache), running on a static scratch array of 64 MiB per device
 * instead of a caller's workspace. The call allocates nothing. A call whose
 * workspace would exceed 64 MiB (coli_moe_workspace_size; about 200 tokens at
 * hidden 6144, inter 2048, 256 experts, top-8) returns COLI_ENOMEM before
 * anything is enqueued. The scratch belongs to the calling thread's current
 * device; the first call on a device looks up its address (make that first
 * call outside graph capture). Every call on one device shares that device's
 * scratch and leaves its contents behind: calls that may overlap on one device
 * (two streams, or two threads) race and must be ordered by the caller. */
COLI_API coli_status coli_moe_layer_fwd_noalloc(const coli_moe_shape* shape, const float* d_x,
                                               int32_t T, const float* d_logits,
                                               const float* d_router_w, const float* d_bias,
                                               const void* const* d_blob_table,
                                               const void* d_shared_blob, float* d_y,
                                               int32_t* d_idx_out, float* d_w_out, int32_t path,
                                               void* stream);

/* ------------------------------------------------------------ expert cache
 * Per-layer LRU of expert blobs in an HBM arena, filled from pinned host
 * memory (practical guide section 二: per-layer LRU; a miss is one read of the
 * whole expert; a read in flight is never issued twice; misses load while
 * resident experts compute; placement changes speed, never the result). */
typedef struct coli_cache_cfg {
    int32_t n_layers;
    int32_t n_experts;          /* routed experts per layer */
    int32_t slots_per_layer;    /* HBM slots per layer, >= top_k of the calls */
    size_t blob_bytes;          /* bytes per expert blob */
    void* d_arena;              /* device, n_layers * slots_per_layer * blob_bytes */
    const void* const* h_pools; /* host array [n_layers] of pinned host pointers, each to
                                   n_experts * blob_bytes; blob e of layer l at
                                   h_pools[l] + e * blob_bytes (layers may share a pool) */
    void* copy_stream;          /* hipStream_t for the host-to-device copies */
} coli_cache_cfg;

typedef struct coli_cache_stats {
    uint64_t hits;              /* lookups of a resident expert (pinned and prefetched ones too) */
    uint64_t misses;            /* lookups that copied the expert */
    uint64_t evictions;
    uint64_t bytes_h2d;         /* every copy: misses, pins and prefetches */
    uint64_t copy_ns;           /* sum of the copies' event-measured durations */
    uint64_t lookups;           /* distinct experts named per ensure, summed */
    uint64_t pin_hits;          /* hits on pinned slots */
    uint64_t pin_loads;         /* copies made to pin an expert */
    uint64_t prefetches;        /* copies started by a prefetch */
    uint64_t prefetch_hits;     /* first lookup of a prefetched expert */
    uint64_t repin_swaps;
} coli_cache_stats;

/* Creates the handle and its per-layer device pointer tables (n_layers *
 * n_experts pointers; entries of non-resident experts are unspecified). The
 * pool pointer array is copied; the pools themselves must outlive the handle.
 * With d_arena and h_pools both NULL the handle only keeps the books (no
 * copies, no events): the placement policy can be simulated without a GPU. */
COLI_API coli_status coli_expert_cache_create(const coli_cache_cfg* cfg, struct coli_expert_cache** out);
COLI_API coli_status coli_expert_cache_destroy(struct coli_expert_cache* cache);

/* Make experts h_ids[0..n) of `layer` resident. Hits refresh their LRU age;
 * each miss evicts the least recently used slot not named in this call
 * (waiting, on the copy stream, for the compute that last read it) and
 * enqueues one host-to-device copy on the copy stream. h_miss_mask[i]
 * (nullable) is set to 1 for a miss. Duplicate ids count once. COLI_EBUSY if
 * n exceeds the layer's slots. Host-side bookkeeping only; never blocks on
 * the GPU. It takes no compute stream: everything it enqueues goes on the
 * cache's copy stream, and the compute stream is joined by
 * coli_expert_cache_wait. If a copy cannot be enqueued the call returns
 * COLI_EHIP with that copy's slot left empty (its expert not resident and not
 * counted as a miss); copies enqueued before it in the same call stand. */
COLI_API coli_status coli_expert_cache_ensure(struct coli_expert_cache* cache, int32_t layer,
                                     const int32_t* h_ids, int32_t n, int32_t* h_miss_mask);

/* Make `compute_stream` wait for the copies enqueued by the last ensure on
 * `layer` (and for its pointer-table update). */
COLI_API coli_status coli_expert_cache_wait(struct coli_expert_cache* cache, int32_t layer,
                                   void* compute_stream);

/* Record that the slots used by the last ensure on `layer` are read by work
 * already enqueued on `compute_stream`; a later eviction waits for it. */
COLI_API coli_status coli_expert_cache_release(struct coli_expert_cache* cache, int32_t layer,
                                      void* compute_stream);

/* Device pointer table [n_experts] of `layer` (valid for resident experts
 * once coli_expert_cache_wait has been called on the stream that reads it). */
COLI_API coli_status coli_expert_cache_table(struct coli_expert_cache* cache, int32_t layer,
                                    const void* const** d_table);

COLI_API coli_status coli_expert_cache_stats(struct coli_expert_cache* cache, coli_cache_stats* out);

/* Forget every resident expert (the next lookups all miss); pins, usage
 * history, heat and stats zeroed. */
COLI_API coli_status coli_expert_cache_reset(struct coli_expert_cache* cache);

/* ------------------------------------------------- learned placement
 * The practical guide's tuning section (section 五): the engine records which
 * experts each layer's tokens are routed to (a usage history), pins the
 * hottest experts so that they are never evicted, lets pinned experts share
 * one memory budget with the LRU, and can swap cold pinned experts for hot ones
 * at safe boundaries from a decaying session heat map, with 25% hysteresis and
 * at most four swaps at a time; and (section 二) a router lookahead applies the
 * next layer's router early and prefetches what it picks. Here the budget is
 * the layer's slots: pinned slots are never chosen as victims, and the rest
 * are the LRU. Placement still changes speed only, never results. */

/* Make h_ids[0..n) the pinned set of `layer` (replacing earlier pins, which
 * become plain LRU entries); members not resident are copied in on the copy
 * stream. Distinct ids count once. COLI_EBUSY if they exceed the slots, or
 * the free slots while a call of the layer is not yet released; nothing
 * changes then. A later ensure that names more unpinned experts than
 * unpinned slots returns COLI_EBUSY, so leave room for a call's experts. */
COLI_API coli_status coli_expert_cache_pin(struct coli_expert_cache* cache, int32_t layer,
                                  const int32_t* h_ids, int32_t n);

/* Usage history: h_counts [n_layers][n_experts] receives, per expert, how many
 * ensure calls named it since create or reset. */
COLI_API coli_status coli_expert_cache_usage(struct coli_expert_cache* cache, uint64_t* h_counts);

/* Pin, in every layer, the `per_layer` experts with the largest counts in
 * h_counts [n_layers][n_experts] (a saved history; NULL = this cache's own
 * usage history); equal counts go to the lower id; experts with count 0 are
 * not pinned. 0 <= per_layer <= slots_per_layer. */
COLI_API coli_status coli_expert_cache_pin_hot(struct coli_expert_cache* cache,
                                      const uint64_t* h_counts, int32_t per_layer);

/* Repin at a safe boundary (no layer call in flight on the host side). Heat:
 * every ensure adds 1 to each expert it names; after the swaps, every heat is
 * multiplied by `decay` (in [0, 1]). Per layer, up to max_swaps times: the
 * coldest pinned expert (equal heat: the higher id) is unpinned (it stays
 * resident as an LRU entry) and the hottest unpinned expert with heat > 0
 * (equal heat: the lower id) is pinned (copied in if needed), provided its
 * heat exceeds (1 + hysteresis) times the cold one's; otherwise the layer
 * stops. The guide's setting is max_swaps 4, hysteresis 0.25. *h_swaps
 * (nullable) receives the number of swaps over all layers. */
COLI_API coli_status coli_expert_cache_repin(struct coli_expert_cache* cache, int32_t max_swaps,
                                    float hysteresis, float decay, int32_t* h_swaps);

/* Prefetch: start copies of the experts h_ids[0..n) of `layer` that are not
 * resident, in order, each into the LRU victim among slots that are not
 * pinned, not named by this request and not held by an unreleased call of the
 * layer; stops when there is none. Experts already resident or in flight are
 * not read again. A prefetched expert counts as a hit when a call names it;
 * that call runs it after coli_expert_cache_wait, like a miss, if the copy may
 * still be in flight. *h_started (nullable) receives the number of copies. */
COLI_API coli_status coli_expert_cache_prefetch(struct coli_expert_cache* cache, int32_t layer,
                                       const int32_t* h_ids, int32_t n, int32_t* h_started);

/* Router lookahead into the cache: route d_x [T][H] with `layer`'s router
 * (d_router_w [E][H], or d_logits [T][E] already computed; d_bias nullable;
 * shape->topp applies), read the picks back to the host (one blocking
 * 4*T*k-byte read) and coli_expert_cache_prefetch them into `layer`. Meant to
 * run with an earlier state of the tokens (the guide applies layer L+1's
 * router to layer L's post-attention state) so that the copies overlap layer
 * L's work. Uses the routing regions of d_ws (coli_moe_workspace_size for
 * shape and T), so it must be ordered with other calls that share d_ws. */
COLI_API coli_status coli_moe_lookahead(const coli_moe_shape* shape, const float* d_x, int32_t T,
                               const float* d_logits, const float* d_router_w,
                               const float* d_bias, struct coli_expert_cache* cache,
                               int32_t layer, int32_t* h_started, void* d_ws, size_t ws_bytes,
                               void* stream);

/* Testing: make the next n host-to-device copies of any expert cache fail with
 * COLI_EHIP before anything is enqueued (n = 0 turns it off). Process-wide.
 * Lets the error path of a failed copy be exercised without a faulty device. */
COLI_API coli_status coli_debug_fail_copies(int32_t n);

/* Testing: log the weight tiles the GEMV kernels stream, so that a test can
 * check that the batch union reads each unique expert's rows once (lbrq.cn
 * article "github一周涨11k⭐️！25GB 内存跑 744B GLM-5.2 模型！", section 三
 * item 4; practical guide section 二). After this call every gate/up and down
 * GEMV launch (coli_moe_expert_ffn, coli_moe_layer_fwd on the GEMV path) has
 * thread 0 of each workgroup that streamed a tile atomically add 1 to
 * *d_count (a device uint32, zeroed by the caller) and, while the old count
 * is below capacity, write a record of four uint32 to d_records[old count]:
 *   blob address bits 0..31, bits 32..63,
 *   pass << 16 | tile   (pass 0: gate/up, a tile being rows [tile * r,
 *                        (tile + 1) * r) of both matrices; pass 1: down,
 *                        rows of the down matrix, clamped to hidden),
 *   r | passes << 16    (r rows per tile: 16 gate/up and 32 down for one
 *                        token, 32 and 64 for batches; passes: how many
 *                        times the workgroup walked those rows, once per
 *                        chunk of up to 4 tokens).
 * The count goes on past capacity, so an overflow shows. The MFMA path is not
 * logged. d_count = nullptr turns the log off (the default); both buffers are
 * the caller's and must outlive the launches that use them. Process-wide, not
 * thread-safe; launches captured into a graph keep the log set at capture.
 * Errors: COLI_EINVAL for capacity < 0, or for a capacity > 0 without
 * d_records. */
COLI_API coli_status coli_debug_read_log(uint32_t* d_count, void* d_records, int32_t capacity);

/* ---------------------------------------------------------- kernel timing
 * Optional HIP-event timing of the library's main kernels, recorded on the
 * stream each kernel runs on. coli_profile_enable(n) pre-creates n event
 * pairs (0 turns timing off and frees them); each timed launch takes the next
 * pair until they run out. coli_profile_summary(name) waits for the recorded
 * events of kernel `name` ("gemv_gateup", "gemv_down", "gemm_gateup",
 * "gemm_down") and returns how many were timed and their total milliseconds.
 * coli_profile_clear() forgets the records and reuses the pairs. */
COLI_API coli_status coli_profile_enable(int32_t max_records);
COLI_API coli_status coli_profile_clear(void);
COLI_API coli_status coli_profile_summary(const char* name, int64_t* count, double* total_ms);

/* Measurement: enqueue on `stream` one more launch of an expert-FFN pass of
 * the last coli_moe_layer_fwd call made with d_ws, which must have been an
 * uncached GEMV-path call (T <= 16, path COLI_PATH_GEMV or AUTO) with the same
 * shape, T, d_blob_table and d_shared_blob. which = 0: the gate/up GEMV (one
 * token: with the routing folded in, which it publishes again into d_ws);
 * 1: the down GEMV. The pass reads and writes d_ws only and recomputes what
 * the call computed, so back-to-back launches of one kernel can be captured in
 * a graph and timed. The caller's y and routing outputs are not touched. */
COLI_API coli_status coli_profile_rerun(const coli_moe_shape* shape, int32_t T,
                                        const void* const* d_blob_table, const void* d_shared_blob,
                                        int32_t which, void* d_ws, size_t ws_bytes, void* stream);

/* Measurement: a read-only streaming kernel over d_src [bytes] (a multiple of
 * 16), for the practical HBM read ceiling of an access pattern. pattern 0:
 * each workgroup of 256 threads reads a contiguous chunk of row_bytes bytes (a
 * multiple of 4096) with 16-byte loads, up to 16 per thread in flight. pattern
 * 1: d_src holds rows of row_bytes bytes (row_bytes / 16 threads per row: a
 * divisor of 256, or 192 for a 3-wave workgroup); each workgroup reads
 * rows_per_wg consecutive rows (a multiple of the rows its threads cover at
 * once), one 16-byte load per thread and row, up to 16 in flight; with
 * row_bytes 3072 and 1024 these are the decode gate/up and down layouts. One 32-bit word per wave goes to d_sink (sink_bytes must hold one
 * per wave of the launch). Enqueued on `stream`. */
COLI_API coli_status coli_read_probe(const void* d_src, size_t bytes, int32_t pattern,
                                     int32_t row_bytes, int32_t rows_per_wg, void* d_sink,
                                     size_t sink_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif
