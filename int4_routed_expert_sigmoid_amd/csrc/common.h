// Internal definitions shared by the HIP translation units of libcoli_moe.
// Not part of the public interface (include/coli_moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <string>

#include "../../include/coli_moe.h"

namespace coli {

// ---------------------------------------------------------------- errors
void set_error(const std::string& msg);
coli_status fail(coli_status code, const std::string& msg);
coli_status hip_fail(hipError_t err, const char* what);

#define COLI_CHECK_HIP(expr)                                   \
    do {                                                       \
        hipError_t _e = (expr);                                \
        if (_e != hipSuccess) return ::coli::hip_fail(_e, #expr); \
    } while (0)

#define COLI_CHECK_LAUNCH(what)                                \
    do {                                                       \
        hipError_t _e = hipGetLastError();                     \
        if (_e != hipSuccess) return ::coli::hip_fail(_e, what);  \
    } while (0)

// ------------------------------------------------------------ blob layout
struct BlobLayout {
    size_t gate_q, up_q, down_q, gate_s, up_s, down_s, bytes;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline BlobLayout blob_layout(int64_t H, int64_t I, int32_t group) {
    BlobLayout L;
    size_t gq = (size_t)I * (size_t)(H / 2), dq = (size_t)H * (size_t)(I / 2);
    size_t gs = (size_t)I * (size_t)(group ? H / group : 1) * 4;
    size_t ds = (size_t)H * (size_t)(group ? I / group : 1) * 4;
    size_t o = 0;
    L.gate_q = o; o = align256(o + gq);
    L.up_q = o;   o = align256(o + gq);
    L.down_q = o; o = align256(o + dq);
    L.gate_s = o; o = align256(o + gs);
    L.up_s = o;   o = align256(o + gs);
    L.down_s = o; o = align256(o + ds);
    L.bytes = o;
    return L;
}

// One unit of GEMV/GEMM work: an expert blob applied to `count` rows of the
// slot list starting at `begin`.
struct WorkItem {
    const uint8_t* blob;
    int32_t begin;
    int32_t count;
};

// ------------------------------------------------------ activation digits
// The GEMV family multiplies int4 weights by activations held as five planes
// of signed base-16 digits per 32-element block: x_c ~= scale_b * X_c with
// scale_b a power of two chosen so that |X_c| <= 2^18, and
// X_c = sum_{p<5} 16^p d_{p,c}, d in [-8, 7]. Every nibble product
// q * d is then exact in a v_dot8_i32_i4 and the per-block integer sum
// sum_c q_c X_c is exact in int32; the only rounding is X_c = rint(x_c/scale_b)
// (relative error <= 2^-18 of the block's largest |x|).
constexpr int kPlanes = 5;
constexpr int kBlock = 32;                 // elements per block (= one 16-byte nibble load)
constexpr int kWordsPerBlock = kPlanes * 4;

__device__ __forceinline__ int dot8(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
}

// sum over 32 columns of q * X for one block: `w` holds the 32 nibbles of
// the weights, `p[0..4]` the digit planes. Exact.
__device__ __forceinline__ int block_dot(const uint4& w, const uint4* p) {
    int a[kPlanes];
#pragma unroll
    for (int i = 0; i < kPlanes; ++i) {
        int acc = dot8(w.x, p[i].x, 0);
        acc = dot8(w.y, p[i].y, acc);
        acc = dot8(w.z, p[i].z, acc);
        acc = dot8(w.w, p[i].w, acc);
        a[i] = acc;
    }
    return a[0] + a[1] * 16 + a[2] * 256 + a[3] * 4096 + a[4] * 65536;
}

// Encode 8 consecutive elements (this thread's quarter of a 32-element block;
// the four quarters are lanes 4i..4i+3 of the wave) into one word per plane.
// Returns the block scale (identical in the four lanes).
__device__ __forceinline__ float encode_quarter(const float v[8], uint32_t words[kPlanes]) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
#pragma unroll
    for (int p = 0; p < kPlanes; ++p) words[p] = 0u;
    if (m == 0.f) return 0.f;
    int ex;
    frexpf(m, &ex);                         // m < 2^ex
    int s = ex - 18;                        // |x| * 2^-s < 2^18
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int X = (int)rintf(ldexpf(v[i], -s));
#pragma unroll
        for (int p = 0; p < kPlanes; ++p) {
            int d = ((X + 8) & 15) - 8;
            X = (X - d) >> 4;
            words[p] |= (uint32_t)(d & 15) << (4 * i);
        }
    }
    return ldexpf(1.0f, s);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ------------------------------------------------- launch entry points
// (host functions implemented in the .hip files; all enqueue on `stream`)
coli_status launch_quantize(const float* w, int64_t rows, int64_t cols, int32_t group,
                            uint8_t* q, float* s, hipStream_t stream);
coli_status launch_router_logits(const float* wr, const float* x, int32_t T, int32_t H,
                                 int32_t E, float* logits, hipStream_t stream);
coli_status launch_route(const float* logits, const float* bias, int32_t T, int32_t E,
                         int32_t k, int32_t* idx, float* w, hipStream_t stream);
size_t union_ws_bytes(int32_t T, int32_t k, int32_t E);
coli_status launch_union(const int32_t* idx, int32_t T, int32_t k, int32_t E, int32_t* counts,
                         int32_t* offsets, int32_t* perm, int32_t* unique, int32_t* n_unique,
                         void* ws, hipStream_t stream);
// Work list from a union: items [max_items], *n_items, rows_tok/rows_out
// [T*k + T]. With a shared blob, item 0 is the shared expert over all T
// tokens (output rows T*k + t). `phase_mask` (nullable, [E]) keeps only
// experts whose mask value equals `phase`.
coli_status launch_plan(const int32_t* offsets, const int32_t* perm,
                        const int32_t* unique, const int32_t* n_unique,
                        const void* const* blob_table, const void* shared_blob, int32_t T,
                        int32_t k, int32_t E, const uint8_t* phase_mask, int32_t phase,
                        WorkItem* items, int32_t* n_items, int32_t* rows_tok, int32_t* rows_out,
                        hipStream_t stream);
coli_status launch_encode(const float* x, int32_t rows, int32_t K, uint32_t* planes, float* scales,
                          hipStream_t stream);
coli_status launch_gemv_ffn(const WorkItem* items, const int32_t* n_items, int32_t max_items,
                            int32_t max_count, const int32_t* rows_tok, const int32_t* rows_out,
                            const uint32_t* xplanes, const float* xscale, uint32_t* hplanes,
                            float* hscale, float* y_rows, int32_t H, int32_t I, int32_t group,
                            hipStream_t stream);
coli_status launch_combine(const float* y_rows, const float* w, int32_t T, int32_t k, int32_t H,
                           int32_t has_shared, float routed_scale, float* y, hipStream_t stream);

}  // namespace coli
