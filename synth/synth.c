/*
 * Seeded synthetic inputs for the int4 routed-expert MoE layer.
 *
 * This module only draws random numbers: weights, activations, router
 * weights, biases and router logits with the shapes and distributions of the
 * workloads. It holds none of the layer's arithmetic (no quantisation, no
 * routing, no union, no FFN), so both the CPU oracle and the GPU path can take
 * their inputs from it without sharing any of the method.
 *
 * Every value is a pure function of (seed, tag, sub0, sub1, index): the
 * counter-based Philox4x32-10 generator of Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3" (SC'11), keyed by
 * (seed, tag) with counter (index_lo, index_hi, sub0, sub1). Any sub-range of
 * any tensor can therefore be regenerated on its own (for example one expert
 * of one layer), in any order and on any number of threads.
 *
 * Normals come from the Box-Muller transform in double precision and are
 * rounded once to float.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

/* Philox4x32 with 10 rounds, as defined in the SC'11 paper. */
void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline void block(uint32_t seed, uint32_t tag, uint32_t sub0, uint32_t sub1,
                         uint64_t i, uint32_t out[4]) {
    uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), sub0, sub1};
    uint32_t key[2] = {seed, tag};
    synth_philox4x32_10(ctr, key, out);
}

/* 53-bit uniform in [0, 1) from two 32-bit words. */
static inline double u53(uint32_t hi, uint32_t lo) {
    uint64_t v = (((uint64_t)hi << 32) | lo) >> 11;
    return (double)v * (1.0 / 9007199254740992.0);
}

/* Standard-normal pair from one Philox block. u1 lies in (0, 1] so log is finite. */
static inline void normal_pair(const uint32_t r[4], double* z0, double* z1) {
    double u1 = 1.0 - u53(r[0], r[1]);
    double u2 = u53(r[2], r[3]);
    double rad = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    *z0 = rad * cos(th);
    *z1 = rad * sin(th);
}

/* out[j] = (float)(mean + std * z[first + j]) for j in [0, n), where z[i] is
 * the i-th standard normal of stream (seed, tag, sub0, sub1). */
void synth_normal_f32(uint32_t seed, uint32_t tag, uint32_t sub0, uint32_t sub1,
                      int64_t first, int64_t n, double mean, double std, float* out) {
    if (n <= 0) return;
    int64_t p_begin = first >> 1, p_end = (first + n + 1) >> 1;
#pragma omp parallel for schedule(static)
    for (int64_t p = p_begin; p < p_end; ++p) {
        uint32_t r[4];
        double z0, z1;
        block(seed, tag, sub0, sub1, (uint64_t)p, r);
        normal_pair(r, &z0, &z1);
        int64_t i0 = 2 * p, i1 = 2 * p + 1;
        if (i0 >= first && i0 < first + n) out[i0 - first] = (float)(mean + std * z0);
        if (i1 >= first && i1 < first + n) out[i1 - first] = (float)(mean + std * z1);
    }
}

/* out[j] = i-th uniform double in [0, 1) of the stream, i = first + j. */
void synth_uniform_f64(uint32_t seed, uint32_t tag, uint32_t sub0, uint32_t sub1,
                       int64_t first, int64_t n, double* out) {
    if (n <= 0) return;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        uint32_t r[4];
        block(seed, tag, sub0, sub1, (uint64_t)(first + j), r);
        out[j] = u53(r[0], r[1]);
    }
}

/* A seeded permutation of 0..n-1 (Fisher-Yates, one uniform per step). */
void synth_permutation(uint32_t seed, uint32_t tag, uint32_t sub0, uint32_t sub1,
                       int32_t n, int32_t* out) {
    for (int32_t i = 0; i < n; ++i) out[i] = i;
    for (int32_t i = n - 1; i > 0; --i) {
        uint32_t r[4];
        block(seed, tag, sub0, sub1, (uint64_t)i, r);
        int32_t j = (int32_t)(u53(r[0], r[1]) * (double)(i + 1));
        if (j > i) j = i;
        int32_t t = out[i]; out[i] = out[j]; out[j] = t;
    }
}

/* Router logits whose top-k is a Plackett-Luce draw from a popularity law:
 * logit[t][e] = ln p[rank[e]] + Gumbel(0,1), where the rank of expert e is
 * perm[e] (0-based) and p[r] is proportional to (r+1)^-s, mixed with a
 * uniform share: p = (1-mix) Zipf(s) + mix / E. Adding Gumbel noise to log
 * probabilities and taking the k largest draws k items without replacement in
 * proportion to p. */
void synth_zipf_gumbel_logits(uint32_t seed, uint32_t tag, uint32_t sub0,
                              int64_t t_first, int64_t T, int32_t E, double s, double mix,
                              const int32_t* perm, float* logits) {
    double* lp = (double*)malloc(sizeof(double) * (size_t)E);
    double z = 0.0;
    for (int32_t r = 0; r < E; ++r) z += pow((double)(r + 1), -s);
    for (int32_t r = 0; r < E; ++r)
        lp[r] = log((1.0 - mix) * pow((double)(r + 1), -s) / z + mix / (double)E);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            uint32_t r[4];
            block(seed, tag, sub0, (uint32_t)(t_first + t), (uint64_t)e, r);
            double u = 1.0 - u53(r[0], r[1]); /* (0, 1] */
            double g = (u >= 1.0) ? -log(-log(1.0 - 1e-17)) : -log(-log(u));
            logits[t * E + e] = (float)(lp[perm[e]] + g);
        }
    }
    free(lp);
}

/* Routing with temporal locality, encoded as logits whose top-k is the chosen
 * set: token 0 draws k experts by popularity (Zipf(s) over ranks perm[e]);
 * every later token keeps each of the previous token's experts with
 * probability keep_p and fills the rest by popularity, without replacement.
 * Chosen experts get logits ~U(hi_lo, hi_hi), the others ~U(lo_lo, lo_hi), so
 * the chosen set is exactly the top-k when hi_lo > lo_hi and the bias is 0.
 * Sequential in t by construction. chosen_out (T*k, nullable) receives the
 * chosen sets in draw order. */
void synth_locality_logits(uint32_t seed, uint32_t tag, uint32_t sub0,
                           int64_t T, int32_t E, int32_t k, double keep_p, double s,
                           const int32_t* perm, double hi_lo, double hi_hi,
                           double lo_lo, double lo_hi, float* logits, int32_t* chosen_out) {
    double* w = (double*)malloc(sizeof(double) * (size_t)E);
    int32_t* prev = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    int32_t* cur = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    for (int32_t e = 0; e < E; ++e) w[e] = pow((double)(perm[e] + 1), -s);
    for (int64_t t = 0; t < T; ++t) {
        uint64_t ctr = 0;
        uint32_t r[4];
        memset(taken, 0, (size_t)E);
        int32_t n = 0;
        if (t > 0) {
            for (int32_t j = 0; j < k; ++j) {
                block(seed, tag, sub0, (uint32_t)t, ctr++, r);
                if (u53(r[0], r[1]) < keep_p) { cur[n++] = prev[j]; taken[prev[j]] = 1; }
            }
        }
        while (n < k) {
            double tot = 0.0;
            for (int32_t e = 0; e < E; ++e) if (!taken[e]) tot += w[e];
            block(seed, tag, sub0, (uint32_t)t, ctr++, r);
            double u = u53(r[0], r[1]) * tot, acc = 0.0;
            int32_t pick = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                acc += w[e];
                pick = e;
                if (u < acc) break;
            }
            cur[n++] = pick;
            taken[pick] = 1;
        }
        for (int32_t e = 0; e < E; ++e) {
            block(seed, tag, sub0, (uint32_t)t, ctr++, r);
            double u = u53(r[0], r[1]);
            double v = taken[e] ? hi_lo + (hi_hi - hi_lo) * u : lo_lo + (lo_hi - lo_lo) * u;
            logits[t * E + e] = (float)v;
        }
        for (int32_t j = 0; j < k; ++j) {
            prev[j] = cur[j];
            if (chosen_out) chosen_out[t * k + j] = cur[j];
        }
    }
    free(w); free(prev); free(cur); free(taken);
}

int synth_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
