// Internal definitions shared by the HIP translation units of libcoli_moe.
// Not part of the public interface (include/coli_moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>
#include <stddef.h>

#include <string>

#include "../../include/coli_moe.h"
#include "profile.h"

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
// int4 rows hold two nibbles per byte. int8 rows hold, for every 32-element
// block, 16 bytes of high nibbles h = q >> 4 (in [-8, 7]) and then 16 bytes of
// low nibbles l = (q & 15) - 8 (in [-8, 7]), so q = 16 h + l + 8 and the int4
// dot-product machinery serves both.
struct BlobLayout {
    size_t gate_q, up_q, down_q, gate_s, up_s, down_s, bytes;
    int32_t wbits;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Gate and up rows of a blob are interleaved in blocks of kGuBlock rows: block
// b of gate, then block b of up, so that a tile of both matrices' rows is one
// contiguous stretch. Row r of gate sits at gate_q + gu_row(r) * row bytes, row
// r of up at up_q + gu_row(r) * row bytes (up_q = gate_q + kGuBlock rows).
constexpr int kGuBlock = 16;
__host__ __device__ inline int64_t gu_row(int64_t r) {
    return (r / kGuBlock) * (2 * kGuBlock) + r % kGuBlock;
}

inline BlobLayout blob_layout(int64_t H, int64_t I, int32_t group, int32_t wbits = 4) {
    BlobLayout L;
    L.wbits = wbits == 8 ? 8 : 4;
    const int64_t div = L.wbits == 8 ? 1 : 2;
    size_t gq = (size_t)I * (size_t)(H / div), dq = (size_t)H * (size_t)(I / div);
    size_t gs = (size_t)I * (size_t)(group ? H / group : 1) * 4;
    size_t ds = (size_t)H * (size_t)(group ? I / group : 1) * 4;
    size_t o = 0;
    L.gate_q = o;                                   // gate and up rows interleaved (gu_row)
    L.up_q = o + (size_t)kGuBlock * (size_t)(H / div);
    o = align256(o + 2 * gq);
    L.down_q = o; o = align256(o + dq);
    L.gate_s = o; o = align256(o + gs);
    L.up_s = o;   o = align256(o + gs);
    L.down_s = o; o = align256(o + ds);
    L.bytes = o;
    return L;
}

// One unit of GEMV/GEMM work: an expert blob applied to rows begin ..
// begin+count-1 of the slot list (rows_tok / rows_out). row0 is rows_out[begin]
// where one-token passes read it (one-token work lists); items of a batch keep
// their expert's first assignment there, unread.
struct WorkItem {
    const uint8_t* blob;
    int32_t begin;
    int32_t count;
    int32_t row0;
};

// One-token routing folded into the gate/up GEMV: the router's first pass
// has written one 64-bit selection code and one sigmoid score per expert;
// every gate/up workgroup selects the top-k itself and derives its own work
// item, and one workgroup publishes the routing and the work list for the
// later passes. codes == nullptr: the work list comes from the router.
struct FusedRoute {
    const uint64_t* codes;      // [E] selection codes
    const float* scores;        // [E] sigmoid scores
    const void* const* table;   // [E] routed expert blobs
    const void* shared;         // shared expert blob or nullptr
    int32_t E, k;
    float topp;
    int32_t* idx;               // [k] routing out (slot order; -1 for dropped slots)
    float* w;                   // [k]
    int32_t* rows_tok;          // [k + 1]
    int32_t* rows_out;          // [k + 1]
    WorkItem* items;            // [1 + k] work list for the down pass
    int32_t* n_items;
};
constexpr int kFusedMaxExperts = 256;   // four selection codes per lane

// Optional log of the weight tiles the GEMV kernels stream (switched on by
// coli_debug_read_log; count == nullptr: off). Thread 0 of every workgroup
// that streamed a tile appends {blob address low word, high word,
// pass << 16 | tile, rows per tile | passes over the rows << 16}; pass 0 is
// the gate/up kernel (a tile: rows of both matrices), 1 the down kernel. The
// count keeps counting past cap, so an overflow shows.
struct ReadLog {
    uint32_t* count;
    uint4* rec;
    int32_t cap;
};

__device__ __forceinline__ void log_read(const ReadLog& rl, const void* blob, int pass, int tile,
                                         int rows, int passes) {
    if (rl.count == nullptr || threadIdx.x != 0) return;
    const uint32_t i = atomicAdd(rl.count, 1u);
    if (i < (uint32_t)rl.cap) {
        const uint64_t b = (uint64_t)blob;
        rl.rec[i] = make_uint4((uint32_t)b, (uint32_t)(b >> 32), ((uint32_t)pass << 16) | (uint32_t)tile,
                               (uint32_t)rows | ((uint32_t)passes << 16));
    }
}

// The log the GEMV launches pass (gemv.hip).
ReadLog read_log_current();

// ------------------------------------------------------ activation digits
// The GEMV family multiplies int4 weights by activations held as four planes
// of signed base-16 digits per 32-element block: x_c ~= scale_b * X_c with
// scale_b = max_c |x_c| / kDigitMax and X_c = rint(x_c / scale_b) written as
// sum_{p<4} 16^p d_{p,c}, d in [-8, 7]. Four such digits cover every integer
// in [-34952, 30583], so |X_c| <= kDigitMax = 30583 always decomposes. Every
// nibble product q * d is then exact in a v_dot8_i32_i4 and the per-block
// integer sum sum_c q_c X_c is exact in int32; the only rounding is that of
// X_c (at most half a step, step = max|x| / 30583 of the block).
constexpr int kPlanes = 4;
constexpr int kDigitMax = 30583;     // 7 * (16^4 - 1) / 15
constexpr int kBlock = 32;                 // elements per block (= one 16-byte nibble load)
constexpr int kWordsPerBlock = kPlanes * 4;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
typedef __attribute__((address_space(1))) const float global_f32;

// Streaming 128-bit load of weight nibbles (read once: non-temporal). The
// pointer is cast to the global address space: blob pointers come from
// tables in memory, and a generic (FLAT) load would also count against the
// LDS wait counter and serialise the prefetching.
__device__ __forceinline__ uint4 ldg128(const uint8_t* p) {
    const u32x4 v = __builtin_nontemporal_load((global_u32x4*)(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Scheduling boundary: the backend's machine scheduler moves nothing across
// it. Loads through const __restrict__ pointers count as invariant, so an
// empty asm statement with a memory clobber does not hold them in place.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Plain global load of one float through a global-address-space pointer.
__device__ __forceinline__ float ldg_f32(const float* p) { return *(global_f32*)(p); }

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
    return a[0] + a[1] * 16 + a[2] * 256 + a[3] * 4096;
}

// One block of weights in registers: 16 bytes of nibbles (int4), or the high
// and the low nibble planes of an int8 block (32 bytes).
template <bool W8>
struct WBlock {
    uint4 v[W8 ? 2 : 1];
};

// Block `ch` of a weight row (row start `row`).
template <bool W8>
__device__ __forceinline__ WBlock<W8> load_wblock(const uint8_t* row, int ch) {
    WBlock<W8> b;
    if constexpr (W8) {
        b.v[0] = ldg128(row + (size_t)ch * 32);
        b.v[1] = ldg128(row + (size_t)ch * 32 + 16);
    } else {
        b.v[0] = ldg128(row + (size_t)ch * 16);
    }
    return b;
}

// sum over the block of q * X: int4 directly; int8 as 16 (h . X) + (l . X) +
// 8 sum(X), with xsum = sum(X) of the block (digit_sum). Exact in int32:
// |q X| <= 128 * 34952 per element.
template <bool W8>
__device__ __forceinline__ int wblock_dot(const WBlock<W8>& w, const uint4* p, int xsum) {
    if constexpr (W8) return 16 * block_dot(w.v[0], p) + block_dot(w.v[1], p) + 8 * xsum;
    else return block_dot(w.v[0], p);
}

// sum of the block's integers X (all-ones weights through the same dot).
__device__ __forceinline__ int digit_sum(const uint4* p) {
    return block_dot(make_uint4(0x11111111u, 0x11111111u, 0x11111111u, 0x11111111u), p);
}

// The intermediate h = silu(g) * u enters the down pass in blocks of 16
// elements (kHBlock), two per 32-column weight block: the same digit-plane
// words (elements 0-15 of a 32-column block in words x and y of each plane,
// 16-31 in z and w), with one scale per half. The gate/up pass encodes h
// itself, and a workgroup of it holds 16 consecutive rows of both matrices.
constexpr int kHBlock = 16;

// sums over the two 16-column halves of a block of q * X. Exact.
__device__ __forceinline__ int2 block_dot_halves(const uint4& w, const uint4* p) {
    int lo[kPlanes], hi[kPlanes];
#pragma unroll
    for (int i = 0; i < kPlanes; ++i) {
        lo[i] = dot8(w.y, p[i].y, dot8(w.x, p[i].x, 0));
        hi[i] = dot8(w.w, p[i].w, dot8(w.z, p[i].z, 0));
    }
    return make_int2(lo[0] + lo[1] * 16 + lo[2] * 256 + lo[3] * 4096,
                     hi[0] + hi[1] * 16 + hi[2] * 256 + hi[3] * 4096);
}

// the halves' sums of the block's integers X
__device__ __forceinline__ int2 digit_sum_halves(const uint4* p) {
    return block_dot_halves(make_uint4(0x11111111u, 0x11111111u, 0x11111111u, 0x11111111u), p);
}

// wblock_dot per 16-column half (xsum: digit_sum_halves of the block)
template <bool W8>
__device__ __forceinline__ int2 wblock_dot_halves(const WBlock<W8>& w, const uint4* p, int2 xsum) {
    if constexpr (W8) {
        const int2 h = block_dot_halves(w.v[0], p), l = block_dot_halves(w.v[1], p);
        return make_int2(16 * h.x + l.x + 8 * xsum.x, 16 * h.y + l.y + 8 * xsum.y);
    } else {
        return block_dot_halves(w.v[0], p);
    }
}

// ------------------------------------------------- wave transpose-reduce
// Sums N partials (N a power of two <= 64) over the 64 lanes of a wave in
// one pass: every stage pairs each lane with a partner in the other half of
// its lane group, keeps half of the values and adds the partner's copy of
// them. Stage partners: lane^32 and lane^16 via v_permlane32/16_swap,
// lane^8 (DPP row_ror:8), lane^7 (DPP row_half_mirror), lane^2 and lane^1
// (DPP quad_perm). Afterwards lane l holds the wave-wide sum of value
// l >> (6 - log2 N).
__device__ __forceinline__ float dpp_f(float v, int ctrl_sel) {
    const int i = __float_as_int(v);
    int r;
    switch (ctrl_sel) {
        case 8: r = __builtin_amdgcn_update_dpp(0, i, 0x128, 0xF, 0xF, false); break;  // row_ror:8
        case 4: r = __builtin_amdgcn_update_dpp(0, i, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
        case 2: r = __builtin_amdgcn_update_dpp(0, i, 0x4E, 0xF, 0xF, false); break;   // quad_perm 2,3,0,1
        default: r = __builtin_amdgcn_update_dpp(0, i, 0xB1, 0xF, 0xF, false); break;  // quad_perm 1,0,3,2
    }
    return __int_as_float(r);
}

// Value of lane partner(l) for the butterfly partners used in this file:
// S = 1, 2 (lane^S, DPP quad_perm), 4 (lane^7, DPP row_half_mirror),
// 8 (lane^8, DPP row_ror:8), 16 (lane^16), 32 (lane^32) via permlane swaps.
// The six partners generate all 64 lanes, so a butterfly over them is a
// full all-reduce.
template <int S>
__device__ __forceinline__ int lane_xchg(int v) {
    if constexpr (S == 32 || S == 16) {
        const auto r = (S == 32) ? __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false)
                                 : __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
        const int lane = threadIdx.x & 63;
        return (int)((lane & S) ? r[0] : r[1]);
    } else {
        return __float_as_int(dpp_f(__int_as_float(v), S));
    }
}

// X = rint(v * inv) clamped to [-kDigitMax, kDigitMax], as its four signed
// base-16 digits (lowest first), each as a 4-bit two's-complement nibble.
__device__ __forceinline__ void digit_nibbles(float v, float inv, uint32_t nib[kPlanes]) {
    int X = (int)rintf(v * inv);
    X = min(max(X, -kDigitMax), kDigitMax);
#pragma unroll
    for (int p = 0; p < kPlanes; ++p) {
        const int d = ((X + 8) & 15) - 8;
        X = (X - d) >> 4;
        nib[p] = (uint32_t)(d & 15);
    }
}

// Encode 8 consecutive elements (this thread's part of a block of 8 * NL
// elements; the NL parts of a block are lanes NL*i .. NL*i + NL - 1 of the
// wave) into one word per plane. Returns the block scale (identical in the NL
// lanes). NL = 4: 32-element blocks of x; NL = 2: 16-element blocks of h.
template <int NL>
__device__ __forceinline__ float encode_octet(const float v[8], uint32_t words[kPlanes]) {
    static_assert(NL == 2 || NL == 4, "blocks of 16 or 32 elements");
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, __int_as_float(lane_xchg<1>(__float_as_int(m))));
    if constexpr (NL == 4) m = fmaxf(m, __int_as_float(lane_xchg<2>(__float_as_int(m))));
#pragma unroll
    for (int p = 0; p < kPlanes; ++p) words[p] = 0u;
    if (m == 0.f) return 0.f;
    const float inv = (float)kDigitMax / m;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t nib[kPlanes];
        digit_nibbles(v[i], inv, nib);
#pragma unroll
        for (int p = 0; p < kPlanes; ++p) words[p] |= nib[p] << (4 * i);
    }
    return m / (float)kDigitMax;
}

// 32-element blocks (x): the four quarters of a block in lanes 4i..4i+3
__device__ __forceinline__ float encode_quarter(const float v[8], uint32_t words[kPlanes]) {
    return encode_octet<4>(v, words);
}

// Wave-wide sum of a double, every lane receiving the total: a butterfly over
// the DPP / permlane partners (lane_xchg), both halves of the value moved by
// each exchange. A fixed order, so the result is the same on every call.
template <int S>
__device__ __forceinline__ double xchg_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)lane_xchg<S>((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)lane_xchg<S>((int)(uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
    v += xchg_f64<32>(v);
    v += xchg_f64<16>(v);
    v += xchg_f64<8>(v);
    v += xchg_f64<4>(v);
    v += xchg_f64<2>(v);
    v += xchg_f64<1>(v);
    return v;
}

// The same encoding of a 16-element block of h spread over the lanes: a
// group of G lanes (G a power of two, aligned) holds the block in lane order,
// NE elements per lane (e0 .. e0 + NE - 1), DUP lanes in a row holding the
// same elements (they compute the same and contribute once), so that the
// first G/2 lanes hold elements 0-7 and the others 8-15. Returns the block
// scale; afterwards lane G*i holds the plane words of elements 0-7 and lane
// G*i + G/2 those of elements 8-15. The maximum and the OR of the nibbles go
// over the DPP / permlane partners (lane_xchg), which generate the group.
template <int G, int DUP, int NE>
__device__ __forceinline__ float encode_h16_lanes(const float (&v)[NE], int e0,
                                                  uint32_t words[kPlanes]) {
    static_assert((G / DUP) * NE == kHBlock, "the group holds one 16-element block");
    static_assert(G >= 4 && G <= 32, "groups of 4 to 32 lanes");
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < NE; ++i) m = fmaxf(m, fabsf(v[i]));
    auto xmax = [&](auto s) {
        constexpr int S = decltype(s)::value;
        if constexpr (S < G) m = fmaxf(m, __int_as_float(lane_xchg<S>(__float_as_int(m))));
    };
    xmax(std::integral_constant<int, 1>{});
    xmax(std::integral_constant<int, 2>{});
    xmax(std::integral_constant<int, 4>{});
    xmax(std::integral_constant<int, 8>{});
    xmax(std::integral_constant<int, 16>{});
    const bool once = ((threadIdx.x & 63) % DUP) == 0;
#pragma unroll
    for (int p = 0; p < kPlanes; ++p) words[p] = 0u;
    if (m != 0.f) {
        // the hardware reciprocal (1 ulp): X may land one step off the
        // correctly rounded quotient, and the clamp keeps it in range
        const float inv = (float)kDigitMax * __builtin_amdgcn_rcpf(m);
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            uint32_t nib[kPlanes];
            digit_nibbles(v[i], inv, nib);
            const int sh = 4 * ((e0 + i) & 7);
#pragma unroll
            for (int p = 0; p < kPlanes; ++p) words[p] |= once ? nib[p] << sh : 0u;
        }
    }
    auto xor_or = [&](auto s) {
        constexpr int S = decltype(s)::value;
        if constexpr (S < G / 2) {
#pragma unroll
            for (int p = 0; p < kPlanes; ++p) words[p] |= (uint32_t)lane_xchg<S>((int)words[p]);
        }
    };
    xor_or(std::integral_constant<int, 1>{});
    xor_or(std::integral_constant<int, 2>{});
    xor_or(std::integral_constant<int, 4>{});
    xor_or(std::integral_constant<int, 8>{});
    return m * (1.0f / (float)kDigitMax);
}

// ------------------------------------------------------- expert selection
// lbrq.cn article "github一周涨11k⭐️！25GB 内存跑 744B GLM-5.2 模型！", section 三
// item 1 and section 四 item 3: sigmoid scores, a selection-only bias, top-k,
// weights normalised over the selected (norm_topk_prob); adaptive expert
// top-p from the practical guide (section 三 and the section 五 tuning table).

// sigmoid in double, rounded once to f32
__device__ __forceinline__ float sigmoid_score(float logit) {
    return (float)(1.0 / (1.0 + exp(-(double)logit)));
}

// Selection order as one unsigned 64-bit number: the key's bits mapped so
// that unsigned order is float order (high word), then the complement of the
// expert id (low word), so a larger key wins and equal keys go to the lower
// id. A -0.0 key is folded to +0.0 first (they compare equal as floats).
// Every valid entry is nonzero; 0 marks an empty or taken entry.
__device__ __forceinline__ uint64_t selection_code(float key, int e) {
    const uint32_t b = __float_as_uint(key + 0.0f);
    const uint32_t o = b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
    return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)e;
}

// Result of select_topk in lane j < k: slot j's expert and its normalised
// weight; kept (wave-uniform) is the number of slots kept by top-p (k without).
struct TopK {
    int my_idx;
    float my_w;
    int kept;
};

template <int S>
__device__ __forceinline__ uint32_t umax_step(uint32_t v) {
    const uint32_t o = (uint32_t)lane_xchg<S>((int)v);
    return o > v ? o : v;
}

// Wave-wide maximum of an unsigned word (butterfly over the DPP / permlane
// partners), returned uniform.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
    v = umax_step<1>(v);
    v = umax_step<2>(v);
    v = umax_step<4>(v);
    v = umax_step<8>(v);
    v = umax_step<16>(v);
    v = umax_step<32>(v);
    return __builtin_amdgcn_readfirstlane(v);
}

// Top-k of one token held by one wave, lane l holding the codes and scores of
// experts l, l+64, ... (code 0: not an expert). Each lane first sorts its codes
// (descending); each of the k rounds then takes the wave-wide maximum of the
// lanes' first codes, as the maximum of their high words (the keys) and, only
// when several lanes share it, of their low words, and the winning lane drops
// its first code. The picks come out in slot order. With 0 < topp < 1 only the
// shortest slot-order prefix whose share of the k selected scores reaches topp
// is kept: slot j is kept iff j == 0 or the share of slots 0..j-1 is below topp
// (the shares only grow, so the kept slots are a prefix). Weights are the
// scores normalised over the kept slots; shares and sums are double, in slot
// order.
template <int EPL>
__device__ __forceinline__ TopK select_topk(uint64_t (&code)[EPL], const float (&score)[EPL],
                                            int k, float topp) {
    const int lane = threadIdx.x & 63;
    uint64_t c[EPL];
    float sc[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        c[i] = code[i];
        sc[i] = score[i];
    }
    // odd-even transposition sort, descending by code
#pragma unroll
    for (int pass = 0; pass < EPL; ++pass)
#pragma unroll
        for (int i = pass & 1; i + 1 < EPL; i += 2) {
            const bool sw = c[i + 1] > c[i];
            const uint64_t a = c[i], b = c[i + 1];
            const float fa = sc[i], fb = sc[i + 1];
            c[i] = sw ? b : a;
            c[i + 1] = sw ? a : b;
            sc[i] = sw ? fb : fa;
            sc[i + 1] = sw ? fa : fb;
        }
    double sum = 0.0;
    double my_prev = 0.0;    // lane j (< k): sum of slots 0..j-1
    float my_sel = 0.f;      // lane j (< k) keeps the score of slot j
    int my_idx = 0;
    for (int j = 0; j < k; ++j) {
        const uint32_t hi = (uint32_t)(c[0] >> 32), lo = (uint32_t)c[0];
        const uint32_t mh = wave_umax(hi);
        uint64_t top = __ballot(hi == mh);
        if (__popcll(top) > 1) {                      // equal keys: the larger low word (lower id)
            const uint32_t ml = wave_umax(hi == mh ? lo : 0u);
            top = __ballot(hi == mh && lo == ml);
        }
        const int src = (int)__builtin_ctzll(top);
        const int e = (int)~(uint32_t)__builtin_amdgcn_readlane((int)lo, src);
        const float s_sel = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc[0]), src));
        if (lane == src) {                            // the winner drops its first code
#pragma unroll
            for (int i = 0; i + 1 < EPL; ++i) {
                c[i] = c[i + 1];
                sc[i] = sc[i + 1];
            }
            c[EPL - 1] = 0;
            sc[EPL - 1] = 0.f;
        }
        if (lane == j) { my_sel = s_sel; my_idx = e; my_prev = sum; }
        sum += (double)s_sel;
    }
    int kept = k;
    double ksum = sum;
    if (topp > 0.f && topp < 1.f) {
        const double share_before = sum == 0.0 ? (double)lane / (double)k : my_prev / sum;
        const bool keep = lane < k && (lane == 0 || share_before < (double)topp);
        kept = __popcll(__ballot(keep));
        if (kept < k) {
            // the kept prefix's sum is the running sum before slot `kept`
            const uint64_t bits = (uint64_t)__double_as_longlong(my_prev);
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bits, kept);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bits >> 32), kept);
            ksum = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
        }
    }
    TopK r;
    r.my_idx = my_idx;
    r.my_w = (ksum == 0.0) ? (float)(1.0 / kept) : (float)((double)my_sel / ksum);
    r.kept = kept;
    return r;
}

template <int S, int N>
__device__ __forceinline__ void transpose_stage(float* v, int lane) {
    constexpr int h = N / 2;
    if constexpr (S >= 16) {
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const auto r = (S == 32)
                ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + h]), false, false)
                : __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + h]), false, false);
            v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    } else {
        const int bit = (S == 4) ? ((lane >> 2) & 1) : ((lane & S) ? 1 : 0);
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const float keep = bit ? v[i + h] : v[i];
            const float give = bit ? v[i] : v[i + h];
            v[i] = keep + dpp_f(give, S);
        }
    }
}

template <int S>
__device__ __forceinline__ float plain_stage(float v) {
    if constexpr (S >= 16) {
        const auto r = (S == 32) ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false)
                                 : __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        return v + dpp_f(v, S);
    }
}

template <int N>
__device__ __forceinline__ float wave_transpose_sum(float (&v)[N]) {
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
    const int lane = threadIdx.x & 63;
    if constexpr (N >= 2) transpose_stage<32, N>(v, lane); else v[0] = plain_stage<32>(v[0]);
    if constexpr (N >= 4) transpose_stage<16, N / 2>(v, lane); else v[0] = plain_stage<16>(v[0]);
    if constexpr (N >= 8) transpose_stage<8, N / 4>(v, lane); else v[0] = plain_stage<8>(v[0]);
    if constexpr (N >= 16) transpose_stage<4, N / 8>(v, lane); else v[0] = plain_stage<4>(v[0]);
    if constexpr (N >= 32) transpose_stage<2, N / 16>(v, lane); else v[0] = plain_stage<2>(v[0]);
    if constexpr (N >= 64) transpose_stage<1, N / 32>(v, lane); else v[0] = plain_stage<1>(v[0]);
    return v[0];
}

template <int N>
__device__ __forceinline__ constexpr int transpose_shift() {
    return N == 64 ? 0 : N == 32 ? 1 : N == 16 ? 2 : N == 8 ? 3 : N == 4 ? 4 : N == 2 ? 5 : 6;
}

// ------------------------------------------------- launch entry points
// (host functions implemented in the .hip files; all enqueue on `stream`)
// gu_rows: the q rows of an expert's gate or up matrix, placed at gu_row(r).
coli_status launch_quantize(const float* w, int64_t rows, int64_t cols, int32_t group,
                            uint8_t* q, float* s, hipStream_t stream, int32_t wbits = 4,
                            bool gu_rows = false);
// Two f32 matrices of the same shape (an expert's gate and up): one launch
// with per-row scales when both have the same alignment, else two.
coli_status launch_quantize_pair(const float* wa, uint8_t* qa, float* sa, const float* wb,
                                 uint8_t* qb, float* sb, int64_t rows, int64_t cols,
                                 int32_t group, hipStream_t stream, int32_t wbits, bool gu_rows);
// FP8 e4m3 codes w8 [rows][cols] with scales [ceil(rows/128)][ceil(cols/128)]
// -> f32 -> int4, through the same quantiser kernels.
coli_status launch_convert_fp8(const uint8_t* w8, const float* scale, int64_t rows, int64_t cols,
                               int32_t group, uint8_t* q, float* s, hipStream_t stream,
                               int32_t wbits = 4, bool gu_rows = false);
// Two matrices of the same shape (an expert's gate and up) in one launch when
// both fit the one-wave-per-row kernel, else one after the other.
coli_status launch_convert_fp8_pair(const uint8_t* w8a, const float* scale_a, uint8_t* qa,
                                    float* sa, const uint8_t* w8b, const float* scale_b,
                                    uint8_t* qb, float* sb, int64_t rows, int64_t cols,
                                    int32_t group, hipStream_t stream, int32_t wbits,
                                    bool gu_rows);
coli_status launch_router_logits(const float* wr, const float* x, int32_t T, int32_t H,
                                 int32_t E, float* logits, hipStream_t stream);
// Router for small batches (T <= kSmallT): logits (when router_w is given)
// and activation encoding, then routing, union and FFN work list.
constexpr int kSmallT = 16;
struct SmallRouterArgs {
    const float* x;            // [T][H]
    const float* router_w;     // [E][H] or NULL
    const float* logits_in;    // [T][E] when router_w is NULL
    const float* bias;         // [E] or NULL
    float* logits_out;         // [T][E] scratch (router_w given)
    int32_t* idx;              // [T][k]
    float* w;                  // [T][k]
    int32_t *counts, *offsets, *perm, *unique, *n_unique;
    WorkItem* items;
    int32_t* n_items;
    int32_t *rows_tok, *rows_out;
    uint32_t* xplanes;
    float* xscale;
    const void* const* table;
    const void* shared_blob;
    const uint8_t* phase_mask; // [E] or NULL: keep only experts whose mask equals `phase`
    int32_t phase;
    int32_t T, E, k, H;
    float topp;                // adaptive expert top-p, active in (0, 1)
    uint64_t* codes;           // [E] or NULL: one token, routing folded into the gate/up pass
    float* scores;             // [E] with codes
    int32_t split;             // GEMV work list: items of at most kItemTokens tokens
};
coli_status launch_router_small(const SmallRouterArgs& a, hipStream_t stream);

// GEMV work items of a small batch take at most kItemTokens tokens: an expert
// that more of the batch's tokens selected becomes several items of
// consecutive tokens. Their workgroups for one tile are a multiple of 8 apart
// in launch order (the grid's tile count is), so they run side by side on one
// XCD and the weight rows cross HBM once; a workgroup walking the rows again
// for its next 4 tokens found them evicted (measured 7.9% above the
// algorithmic bytes).
constexpr int kItemTokens = 4;
// Work items at most, items split so (n = T * k assignments; shared: the
// shared expert's items too).
inline int64_t split_items_bound(int64_t E, int64_t T, int64_t k, bool shared) {
    const int64_t n = T * k;
    return (E < n ? E : n) + n / kItemTokens + (shared ? (T + kItemTokens - 1) / kItemTokens : 0);
}

coli_status launch_route(const float* logits, const float* bias, int32_t T, int32_t E,
                         int32_t k, float topp, int32_t* idx, float* w, hipStream_t stream);
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
// Digit planes of x [rows_idx[r]] (K = hidden) into planes [rows_idx[r]] for
// the rows a work list reads, up to max_count tokens per item.
coli_status launch_encode_items(const WorkItem* items, const int32_t* n_items, int32_t max_items,
                                int32_t max_count, const int32_t* rows_idx, const float* x,
                                int32_t K, uint32_t* planes, float* scales, hipStream_t stream);

// Prefill split: with the MFMA path chosen automatically, an expert with at
// most this many tokens runs on the GEMV family instead of MFMA tiles.
constexpr int kGemvMaxTokens = 4;
// gate/up then down GEMV over a work list. The gate/up pass writes h =
// silu(g) * u of every (item, token) row it computes as digit planes of
// 16-element blocks: hplanes [rows][I/32][16] u32 (the words of a 32-column
// block, kHBlock), hscale [rows][I/32][2]; the down pass reads them.
// passes: kPassGateUp and/or kPassDown.
constexpr int kPassGateUp = 1, kPassDown = 2, kPassBoth = 3;
coli_status launch_gemv_ffn(const WorkItem* items, const int32_t* n_items, int32_t max_items,
                            int32_t max_count, const int32_t* rows_tok, const int32_t* rows_out,
                            const uint32_t* xplanes, const float* xscale, uint32_t* hplanes,
                            float* hscale, float* y_rows, int32_t H, int32_t I, int32_t group,
                            int32_t wbits, const FusedRoute& fr, hipStream_t stream,
                            int passes = kPassBoth);
// y [T][H] = shared row + rs * sum_j w[t][j] * y_rows[t*k + j] in slot order;
// with idx (nullable) given, slots whose index is negative (dropped by top-p)
// add nothing.
coli_status launch_combine(const float* y_rows, const float* w, const int32_t* idx, int32_t T,
                           int32_t k, int32_t H, int32_t has_shared, float routed_scale, float* y,
                           hipStream_t stream);

}  // namespace coli
