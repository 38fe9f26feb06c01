/*
 * CPU oracle for the int4 routed-expert MoE layer with a sigmoid router.
 *
 * TEST INFRASTRUCTURE ONLY. Plain, slow, scalar C99 with double-precision
 * accumulation, written to be checked against the pages by eye. Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no source, header, table or helper with the GPU library.
 *
 * Pages cited (titles as published):
 *  [HF]  "jlnsrk/GLM-5.2-colibri-int4" (Hugging Face model card): container
 *        format (U8 packed int4 nibbles + F32 per-row scales) and the
 *        conversion note (FP8 e4m3 with 128 x 128 block scales -> f32 ->
 *        int4, np.rint matching the engine's lrintf).
 *  [P4]  "github一周涨11k⭐️！25GB 内存跑 744B GLM-5.2 模型！": section 三
 *        items 1 (sigmoid router, 8 of 256 experts per token) and 4
 *        (batch-union MoE); section 四 item 3 (DeepSeek-V3 aux-loss-free
 *        bias, routing and scaling semantics reproduced exactly).
 *  [P5]  "colibrì 實戰指南：以純 C 引擎在消費級硬體上串流運行 744B MoE 模型":
 *        section 一 (~19 MB per int4 expert, ~11 GB routed experts per
 *        token), section 二 (route -> union -> place -> overlapped execute
 *        -> learn; gate/up/down stored adjacently; batch union reads each
 *        unique expert once; placement never changes routing or precision),
 *        section 三 (gs64 group scales recommended over per-row).
 *  [P2]  "解密GLM-5.2-colibri-int4-with-int8-mtp…": config.json values
 *        (256 routed + 1 shared experts, num_experts_per_tok 8,
 *        scoring_func sigmoid, norm_topk_prob true).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - scale = max|w| / 7 over the row (or 64-group), q = rint(w / scale)
 *    with float division and round-half-even, clamped to [-8, 7]; an
 *    all-zero row or group has scale 0 and q = 0.
 *  - nibbles are two's complement; column 2i in bits 0-3, 2i+1 in bits 4-7.
 *  - gs64 groups run along the input (reduction) axis; scales [rows][cols/64].
 *  - sigmoid in double, rounded once to float; the bias enters selection only;
 *    equal keys go to the lower expert index; weights are the unbiased
 *    scores normalised over the k selected (sum in slot order, double).
 *  - activation is SwiGLU: h = silu(gate x) * (up x), y = down h.
 *  - the routed-scale factor rs multiplies the routed sum at the combine; the
 *    shared expert has weight 1.
 *  - adaptive expert top-p keeps the shortest key-order prefix of the k
 *    selected whose share of their scores reaches p, renormalised over it.
 */
#ifndef COLI_ORACLE_H
#define COLI_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Pointers to the six parts of one quantised expert (host memory). gate and up
 * are [inter][hidden/2] bytes, down is [hidden][inter/2] (int4), or [inter][hidden]
 * and [hidden][inter] signed bytes (int8); the scales are one float per row
 * (group 0) or per 64 consecutive inputs of a row (group 64). */
typedef struct oracle_expert {
    const uint8_t* gate_q;
    const uint8_t* up_q;
    const uint8_t* down_q;
    const float* gate_s;
    const float* up_s;
    const float* down_s;
    int32_t bits;          /* 4: packed nibbles (0 means 4 as well); 8: one signed byte per weight */
} oracle_expert;

/* Quantise w [rows][cols] to packed nibbles q [rows][cols/2] and scales s.
 * group is 0 (one scale per row) or 64 (one per 64 consecutive columns).
 * Returns 0, or -1 for bad arguments (cols odd, cols % 64 != 0 with group 64). */
int oracle_quantize_int4(const float* w, int64_t rows, int64_t cols, int32_t group,
                         uint8_t* q, float* s);

/* int8 codec (the MTP head must be int8): scale = max|w| / 127 per row or
 * 64-group, q = rint(w / scale) half-even, clamped to [-128, 127]; q
 * [rows][cols] signed bytes. Returns 0 or -1. */
int oracle_quantize_int8(const float* w, int64_t rows, int64_t cols, int32_t group, int8_t* q,
                         float* s);
void oracle_dequantize_int8(const int8_t* q, const float* s, int64_t rows, int64_t cols,
                            int32_t group, double* out);

/* The float value a stored nibble stands for, in double: q * scale. */
void oracle_dequantize_int4(const uint8_t* q, const float* s, int64_t rows, int64_t cols,
                            int32_t group, double* out);

/* FP8 -> f32 -> int4 conversion ([HF] conversion note). The value of one
 * OCP e4m3 byte (NaN for the two NaN codes). */
double oracle_fp8_e4m3_value(uint8_t b);

/* w [rows][cols] = e4m3(w8[r][c]) * scale[r/128][c/128] rounded once to f32;
 * scale is row-major [ceil(rows/128)][ceil(cols/128)]. Returns 0 or -1. */
int oracle_fp8_block_dequant(const uint8_t* w8, const float* scale, int64_t rows, int64_t cols,
                             float* w);

/* The converter: oracle_fp8_block_dequant, then oracle_quantize_int4. */
int oracle_convert_fp8_int4(const uint8_t* w8, const float* scale, int64_t rows, int64_t cols,
                            int32_t group, uint8_t* q, float* s);

/* logits[t][e] = (float) sum_j (double) wr[e][j] * (double) x[t][j]. */
void oracle_router_logits(const float* wr, const float* x, int32_t T, int32_t H, int32_t E,
                          float* logits);

/* Sigmoid routing: idx[t][0..k) in descending key order, w[t][0..k) normalised.
 * bias may be NULL (zero). Returns 0, or -1 for bad arguments. */
int oracle_route(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                 int32_t* idx, float* w);

/* The same with the adaptive expert top-p p in [0, 1]: for 0 < p < 1 only the
 * shortest prefix of the k slots whose share of the selected scores reaches p
 * is kept, renormalised; dropped slots get idx -1 and w 0. p = 0 or 1 is
 * oracle_route. Returns 0, or -1 for bad arguments (p outside [0, 1]). */
int oracle_route_topp(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                      float p, int32_t* idx, float* w);

/* Batch union of the T*k assignments a = t*k + j: counts[E], offsets[E+1]
 * (exclusive prefix sum), perm[T*k] (assignments grouped by expert, ascending
 * within each group), unique[n] (experts with counts > 0, ascending).
 * Negative entries are slots dropped by top-p: they belong to no expert, and
 * offsets[E] counts only the others. Entries >= E are an error (-1). */
int oracle_union(const int32_t* idx, int32_t T, int32_t k, int32_t E, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* unique, int32_t* n_unique);

/* One token through one expert: y[H] = down (silu(gate x) * (up x)), double. */
void oracle_expert_ffn(const oracle_expert* ex, int32_t H, int32_t I, int32_t group,
                       const float* x, double* y);

/* Unweighted per-assignment outputs for the union: for each unique expert e
 * and each assignment a in its segment, y_assign[a][H] = FFN_e(x[a / k]). */
int oracle_expert_ffn_union(const oracle_expert* experts, int32_t H, int32_t I, int32_t group,
                            const float* x, int32_t T, int32_t k, const int32_t* offsets,
                            const int32_t* perm, const int32_t* unique, int32_t n_unique,
                            double* y_assign);

/* Whole layer for T tokens, with the adaptive expert top-p topp (0 = fixed
 * top-k, as in oracle_route_topp). Exactly one of logits [T][E] and wr [E][H] is
 * non-NULL. shared may be NULL (no shared expert). y [T][H] float; y64 (nullable)
 * receives the double result before its rounding; idx/w (nullable) receive
 * the routing. Returns 0 or -1. */
int oracle_layer(int32_t H, int32_t I, int32_t E, int32_t k, int32_t group, float routed_scale,
                 float topp, const float* x, int32_t T, const float* logits, const float* wr,
                 const float* bias, const oracle_expert* experts, const oracle_expert* shared,
                 float* y, double* y64, int32_t* idx, float* w);

/* Threads the oracle's parallel loops use (1 without OpenMP). */
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
