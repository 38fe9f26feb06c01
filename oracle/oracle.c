/*
 * CPU oracle for the int4 routed-expert MoE layer. TEST INFRASTRUCTURE ONLY:
 * see oracle.h for the pages followed and the readings taken where they are
 * silent. Scalar C99, double accumulation, no blocking, fusion or reordering
 * beyond what each step's definition states.
 */
#include "oracle.h"

#include <fenv.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the OpenMP loops that follow (n >= 1); changes no result, since
 * every output element is summed by one thread in its stated order. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------- quantiser
 * [HF] container: each quantised weight is a U8 tensor of packed int4 nibbles
 * plus an F32 scale per row; the conversion rounds with np.rint, matching the
 * engine's lrintf (round half to even). [P5] section 三: gs64 group scales.
 * Scale max|w|/7 and the clamp to [-8, 7] are the stated reading. */

static int8_t quant_one(float w, float scale) {
    if (scale == 0.0f) return 0;
    float v = rintf(w / scale);          /* float division, nearest-even */
    if (v > 7.0f) v = 7.0f;
    if (v < -8.0f) v = -8.0f;
    return (int8_t)v;
}

int oracle_quantize_int4(const float* w, int64_t rows, int64_t cols, int32_t group,
                         uint8_t* q, float* s) {
    if (rows < 0 || cols <= 0 || (cols & 1)) return -1;
    if (group != 0 && group != 64) return -1;
    if (group == 64 && cols % 64) return -1;
    if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
    int64_t span = group ? group : cols;          /* columns sharing one scale */
    int64_t per_row = cols / span;
    for (int64_t r = 0; r < rows; ++r) {
        const float* wr = w + r * cols;
        uint8_t* qr = q + r * (cols / 2);
        for (int64_t g = 0; g < per_row; ++g) {
            float m = 0.0f;
            for (int64_t c = g * span; c < (g + 1) * span; ++c) {
                float a = fabsf(wr[c]);
                if (a > m) m = a;
            }
            float scale = m / 7.0f;
            s[r * per_row + g] = scale;
            for (int64_t c = g * span; c < (g + 1) * span; c += 2) {
                int8_t lo = quant_one(wr[c], scale);
                int8_t hi = quant_one(wr[c + 1], scale);
                qr[c / 2] = (uint8_t)(((uint8_t)lo & 0x0F) | (((uint8_t)hi & 0x0F) << 4));
            }
        }
    }
    return 0;
}

/* Signed value of nibble c of a packed row (two's complement, low nibble first). */
static int nibble(const uint8_t* row, int64_t c) {
    int v = (c & 1) ? (row[c >> 1] >> 4) : (row[c >> 1] & 0x0F);
    return v >= 8 ? v - 16 : v;
}

/* ------------------------------------------------------- int8 codec
 * [P5] section 二 and the int8-MTP page: the MTP head must be int8 (an int4
 * head's draft acceptance collapses); the converter's options include 8-bit
 * tensors. The pages give no int8 formula; the reading mirrors the int4 rule
 * with 127 in place of 7: scale = max|w| / 127 per row or 64-group (float
 * division), q = rint(w / scale) half-to-even, clamped to [-128, 127], scale 0
 * gives q = 0; q is stored one signed byte per weight, row-major. */
static int8_t quant_one8(float w, float scale) {
    if (scale == 0.0f) return 0;
    float v = rintf(w / scale);
    if (v > 127.0f) v = 127.0f;
    if (v < -128.0f) v = -128.0f;
    return (int8_t)v;
}

int oracle_quantize_int8(const float* w, int64_t rows, int64_t cols, int32_t group, int8_t* q,
                         float* s) {
    if (rows < 0 || cols <= 0) return -1;
    if (group != 0 && group != 64) return -1;
    if (group == 64 && cols % 64) return -1;
    if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
    int64_t span = group ? group : cols;
    int64_t per_row = cols / span;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < per_row; ++g) {
            float m = 0.0f;
            for (int64_t c = g * span; c < (g + 1) * span; ++c)
                if (fabsf(w[r * cols + c]) > m) m = fabsf(w[r * cols + c]);
            float scale = m / 127.0f;
            s[r * per_row + g] = scale;
            for (int64_t c = g * span; c < (g + 1) * span; ++c)
                q[r * cols + c] = quant_one8(w[r * cols + c], scale);
        }
    return 0;
}

/* Stored integer of weight (r, c) of a matrix with `cols` columns: a nibble
 * (bits 4) or a signed byte (bits 8). */
static int qval(const uint8_t* q, int64_t r, int64_t c, int64_t cols, int bits) {
    if (bits == 8) return (int)(int8_t)q[r * cols + c];
    return nibble(q + r * (cols / 2), c);
}

static double scale_of(const float* s, int64_t r, int64_t c, int64_t cols, int32_t group) {
    if (group == 0) return (double)s[r];
    return (double)s[r * (cols / group) + c / group];
}

void oracle_dequantize_int4(const uint8_t* q, const float* s, int64_t rows, int64_t cols,
                            int32_t group, double* out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = (double)nibble(q + r * (cols / 2), c) * scale_of(s, r, c, cols, group);
}

void oracle_dequantize_int8(const int8_t* q, const float* s, int64_t rows, int64_t cols,
                            int32_t group, double* out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = (double)q[r * cols + c] * scale_of(s, r, c, cols, group);
}

/* ------------------------------------------------------- FP8 converter
 * [HF] conversion note: the container was made from the FP8 checkpoint by
 * FP8 (e4m3, one scale factor per 128 x 128 block) -> f32 -> int4, rounding
 * with np.rint. The e4m3 layout is the OCP 8-bit float E4M3: 1 sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes the
 * subnormals m * 2^-9; there is no infinity, and S.1111.111 is NaN. Reading:
 * the block of w[r][c] is (r / 128, c / 128) in a row-major scale array of
 * ceil(rows/128) x ceil(cols/128) floats, and w = e4m3 value times the block's
 * scale, one f32 rounding of the exact product. */
double oracle_fp8_e4m3_value(uint8_t b) {
    const int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);                  /* subnormal: m/8 * 2^-6 */
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

int oracle_fp8_block_dequant(const uint8_t* w8, const float* scale, int64_t rows, int64_t cols,
                             float* w) {
    if (rows < 0 || cols < 0) return -1;
    const int64_t sc_cols = (cols + 127) / 128;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            double v = oracle_fp8_e4m3_value(w8[r * cols + c]);
            double f = (double)scale[(r / 128) * sc_cols + c / 128];
            w[r * cols + c] = (float)(v * f);      /* exact in double, one rounding */
        }
    return 0;
}

int oracle_convert_fp8_int4(const uint8_t* w8, const float* scale, int64_t rows, int64_t cols,
                            int32_t group, uint8_t* q, float* s) {
    if (rows < 0 || cols < 0) return -1;
    float* w = (float*)malloc(sizeof(float) * ((size_t)(rows * cols) + 1));
    if (!w) return -1;
    int rc = oracle_fp8_block_dequant(w8, scale, rows, cols, w);
    if (!rc) rc = oracle_quantize_int4(w, rows, cols, group, q, s);
    free(w);
    return rc;
}

/* ---------------------------------------------------------------- router
 * [P5] section 一/二 and [HF]: the router stays F32. Logits accumulate in
 * double and are rounded once. */
void oracle_router_logits(const float* wr, const float* x, int32_t T, int32_t H, int32_t E,
                          float* logits) {
    for (int32_t t = 0; t < T; ++t)
        for (int32_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int32_t j = 0; j < H; ++j) acc += (double)wr[(int64_t)e * H + j] * (double)x[(int64_t)t * H + j];
            logits[(int64_t)t * E + e] = (float)acc;
        }
}

/* [P4] section 三 item 1: a DeepSeek-V3-style sigmoid router picks 8 of 256
 * experts per token. [P4] section 四 item 3: the aux-loss-free bias adjusts
 * selection; routing, selection and scaling are reproduced exactly. [P2]:
 * scoring_func sigmoid, norm_topk_prob true.
 *
 * Adaptive expert top-p ([P5] section 三, where it is the recommended setting
 * for disk-bound machines at 0.7, and the section 五 tuning table: an
 * adaptive, lossy expert top-p that reads 30-40% fewer expert bytes). The
 * pages give no formula; the reading taken here: the k experts are selected
 * as above, then the shortest prefix of them in key (slot) order whose share
 * of the k selected scores reaches p is kept; its weights are its scores
 * normalised over the kept prefix (the same rule as for the k, applied to
 * fewer experts), and the dropped slots get index -1 and weight 0. The share
 * of the first j+1 slots is (s_0 + ... + s_j) / (s_0 + ... + s_{k-1}), both
 * sums in double in slot order, compared with p in double; it is (j+1)/k when
 * every selected score is 0. p = 0 or p >= 1 keeps all k (fixed top-k). */
int oracle_route_topp(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                      float p, int32_t* idx, float* w) {
    if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
    if (!(p >= 0.0f && p <= 1.0f)) return -1;                  /* NaN too */
    const int adaptive = p > 0.0f && p < 1.0f;
    float* score = (float*)malloc(sizeof(float) * (size_t)E);
    float* key = (float*)malloc(sizeof(float) * (size_t)E);
    unsigned char* used = (unsigned char*)malloc((size_t)E);
    if (!score || !key || !used) { free(score); free(key); free(used); return -1; }
    for (int32_t t = 0; t < T; ++t) {
        const float* l = logits + (int64_t)t * E;
        for (int32_t e = 0; e < E; ++e) {
            score[e] = (float)(1.0 / (1.0 + exp(-(double)l[e])));   /* sigmoid, one rounding */
            key[e] = score[e] + (bias ? bias[e] : 0.0f);            /* float add */
            used[e] = 0;
        }
        /* selection: k passes, each taking the largest remaining key; the
         * strict > keeps the lowest index among equal keys */
        int32_t* it = idx + (int64_t)t * k;
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (used[e]) continue;
                if (best < 0 || key[e] > key[best]) best = e;
            }
            used[best] = 1;
            it[j] = best;
        }
        /* sum of the k selected unbiased scores, in slot order */
        double sum = 0.0;
        for (int32_t j = 0; j < k; ++j) sum += (double)score[it[j]];
        /* adaptive top-p: the number of slots kept */
        int32_t kept = k;
        if (adaptive) {
            double cum = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                cum += (double)score[it[j]];
                double share = (sum == 0.0) ? (double)(j + 1) / (double)k : cum / sum;
                if (share >= (double)p) { kept = j + 1; break; }
            }
        }
        /* normalised weights over the kept slots */
        double ksum = 0.0;
        for (int32_t j = 0; j < kept; ++j) ksum += (double)score[it[j]];
        for (int32_t j = 0; j < k; ++j) {
            float* wj = &w[(int64_t)t * k + j];
            if (j >= kept) { it[j] = -1; *wj = 0.0f; continue; }
            *wj = (ksum == 0.0) ? (float)(1.0 / kept) : (float)((double)score[it[j]] / ksum);
        }
    }
    free(score); free(key); free(used);
    return 0;
}

int oracle_route(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                 int32_t* idx, float* w) {
    return oracle_route_topp(logits, bias, T, E, k, 0.0f, idx, w);
}

/* ----------------------------------------------------------------- union
 * [P4] section 三 item 4 and [P5] section 二: positions of a batch that hit
 * the same expert are merged, so each unique expert is read once and applied
 * to all of its positions. */
int oracle_union(const int32_t* idx, int32_t T, int32_t k, int32_t E, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* unique, int32_t* n_unique) {
    if (T < 0 || k <= 0 || E <= 0) return -1;
    int64_t n = (int64_t)T * k;
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t a = 0; a < n; ++a) {
        if (idx[a] >= E) return -1;
        if (idx[a] < 0) continue;                 /* a slot dropped by top-p */
        counts[idx[a]] += 1;
    }
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    if (!fill) return -1;
    for (int64_t a = 0; a < n; ++a) {
        int32_t e = idx[a];
        if (e < 0) continue;
        perm[offsets[e] + fill[e]] = (int32_t)a;
        fill[e] += 1;
    }
    free(fill);
    int32_t u = 0;
    for (int32_t e = 0; e < E; ++e)
        if (counts[e] > 0) unique[u++] = e;
    *n_unique = u;
    return 0;
}

/* ------------------------------------------------------------ expert FFN
 * [P5] section 二: an expert is three matrices (gate, up, down) stored
 * adjacently. SwiGLU: h_r = silu(g_r) * u_r with g = gate x, u = up x; then
 * y = down h. Each product term is dequantised (nibble * scale) in double. */
void oracle_expert_ffn(const oracle_expert* ex, int32_t H, int32_t I, int32_t group,
                       const float* x, double* y) {
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    const int bits = ex->bits == 8 ? 8 : 4;
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < I; ++r) {
        double g = 0.0, u = 0.0;
        for (int32_t c = 0; c < H; ++c) {
            g += (double)qval(ex->gate_q, r, c, H, bits) * scale_of(ex->gate_s, r, c, H, group) * (double)x[c];
            u += (double)qval(ex->up_q, r, c, H, bits) * scale_of(ex->up_s, r, c, H, group) * (double)x[c];
        }
        h[r] = g / (1.0 + exp(-g)) * u;
    }
#pragma omp parallel for schedule(static)
    for (int32_t c = 0; c < H; ++c) {
        double acc = 0.0;
        for (int32_t r = 0; r < I; ++r)
            acc += (double)qval(ex->down_q, c, r, I, bits) * scale_of(ex->down_s, c, r, I, group) * h[r];
        y[c] = acc;
    }
    free(h);
}

int oracle_expert_ffn_union(const oracle_expert* experts, int32_t H, int32_t I, int32_t group,
                            const float* x, int32_t T, int32_t k, const int32_t* offsets,
                            const int32_t* perm, const int32_t* unique, int32_t n_unique,
                            double* y_assign) {
    if (H <= 0 || I <= 0 || T < 0 || k <= 0) return -1;
    for (int32_t i = 0; i < n_unique; ++i) {
        int32_t e = unique[i];
        for (int32_t p = offsets[e]; p < offsets[e + 1]; ++p) {
            int32_t a = perm[p];
            oracle_expert_ffn(&experts[e], H, I, group, x + (int64_t)(a / k) * H,
                              y_assign + (int64_t)a * H);
        }
    }
    return 0;
}

/* ----------------------------------------------------------------- layer
 * [P5] section 二: per token and layer, route -> union -> (placement) ->
 * execute. The combine sums the routed outputs in slot order weighted by
 * the normalised weights, scales that sum by rs, and adds the shared expert
 * (weight 1) — [P4] section 四 item 3 asks for the scaling semantics to be
 * reproduced; rs defaults to 1. Slots dropped by the adaptive top-p (index
 * -1) have no expert and add nothing. */
int oracle_layer(int32_t H, int32_t I, int32_t E, int32_t k, int32_t group, float routed_scale,
                 float topp, const float* x, int32_t T, const float* logits, const float* wr,
                 const float* bias, const oracle_expert* experts, const oracle_expert* shared,
                 float* y, double* y64, int32_t* idx_out, float* w_out) {
    if (H <= 0 || I <= 0 || E <= 0 || k <= 0 || k > E || T < 0) return -1;
    if ((logits == NULL) == (wr == NULL)) return -1;
    int rc = -1;
    int64_t n = (int64_t)T * k;
    float* lg = (float*)malloc(sizeof(float) * ((size_t)T * E + 1));
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * ((size_t)n + 1));
    float* w = (float*)malloc(sizeof(float) * ((size_t)n + 1));
    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * ((size_t)E + 1));
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * ((size_t)n + 1));
    int32_t* unique = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    double* ya = (double*)malloc(sizeof(double) * ((size_t)n * H + 1));
    double* ys = (double*)malloc(sizeof(double) * (size_t)H);
    int32_t n_unique = 0;
    if (!lg || !idx || !w || !counts || !offsets || !perm || !unique || !ya || !ys) goto done;
    /* rows of slots without an expert (dropped by top-p) hold NaN, so that
     * using one would show in the result */
    for (int64_t i = 0; i < n * H; ++i) ya[i] = NAN;

    if (logits) memcpy(lg, logits, sizeof(float) * (size_t)T * E);
    else oracle_router_logits(wr, x, T, H, E, lg);
    if (oracle_route_topp(lg, bias, T, E, k, topp, idx, w)) goto done;
    if (oracle_union(idx, T, k, E, counts, offsets, perm, unique, &n_unique)) goto done;
    if (oracle_expert_ffn_union(experts, H, I, group, x, T, k, offsets, perm, unique, n_unique, ya))
        goto done;
    for (int32_t t = 0; t < T; ++t) {
        if (shared) oracle_expert_ffn(shared, H, I, group, x + (int64_t)t * H, ys);
        for (int32_t c = 0; c < H; ++c) {
            double routed = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                if (idx[(int64_t)t * k + j] < 0) continue;      /* dropped by top-p */
                routed += (double)w[(int64_t)t * k + j] * ya[((int64_t)t * k + j) * H + c];
            }
            double v = (shared ? ys[c] : 0.0) + (double)routed_scale * routed;
            y[(int64_t)t * H + c] = (float)v;
            if (y64) y64[(int64_t)t * H + c] = v;
        }
    }
    if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)n);
    if (w_out) memcpy(w_out, w, sizeof(float) * (size_t)n);
    rc = 0;
done:
    free(lg); free(idx); free(w); free(counts); free(offsets); free(perm); free(unique);
    free(ya); free(ys);
    return rc;
}
