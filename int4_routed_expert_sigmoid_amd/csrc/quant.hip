// int4 quantiser (the container rule of the model card "jlnsrk/GLM-5.2-colibri-int4":
// packed int4 nibbles + F32 scales, values rounded half-to-even as np.rint /
// lrintf do; gs64 group scales from the practical guide's section 三), and the
// FP8 converter of the same card's conversion note (e4m3 codes with one scale
// per 128 x 128 block -> f32 -> int4), which feeds the same kernels.
//
// scale = max|w| / 7 (float division) per row or per 64 consecutive columns,
// q = rint(w / scale) (float division, nearest-even), clamped to [-8, 7];
// scale 0 gives q = 0. Each thread owns 8 consecutive columns, i.e. one
// 32-bit word of packed output.
#include "common.h"
#include "quant.h"

namespace coli {
namespace {

// q = rint(v / scale) with IEEE division, clamped to [QLO, QHI]. The quotient
// is first formed as t = v * inv with inv = 1/scale correctly rounded. With
// |v / scale| <= 128 (int8; <= 8 for int4), t lies within 128 * 2^-23 = 2^-16
// of the exact quotient (2^-20 for int4), and the correctly rounded quotient
// within half an ulp (2^-17) of it, so rint(t) can differ from rint of the
// correctly rounded quotient only when t lies within 2^-15 (int4: 2^-19) of a
// half-integer. The window used is 2^-14, twice the wider bound: such values
// (and non-finite t, e.g. from a subnormal scale) take the division.
template <int QLO, int QHI>
__device__ __forceinline__ int quant_q(float v, float scale, float inv) {
    const float t = v * inv;
    float r = rintf(t);
    if (!(fabsf(fabsf(t - r) - 0.5f) > 0x1p-14f)) r = rintf(__fdiv_rn(v, scale));
    return (int)fminf(fmaxf(r, (float)QLO), (float)QHI);
}

// rint(t) of quant_q without its division, clamped, and whether the word
// needs the division: |t - rint(t)| within the window of a half-integer, or t
// not finite (the comparison fails for NaN). Same window and same rounding as
// quant_q, so a word built from these equals one built from quant_q whenever
// no element is flagged.
template <int QLO, int QHI>
__device__ __forceinline__ int quant_fast(float v, float inv, bool& near) {
    const float t = v * inv;
    const float r = rintf(t);
    near |= !(fabsf(t - r) < 0.5f - 0x1p-14f);
    return (int)__builtin_amdgcn_fmed3f(r, (float)QLO, (float)QHI);
}

// int4: 8 nibbles of one output word. The division is taken once per word,
// and only for words with an element near a half-integer quotient: with
// |v / scale| <= 7 (1 + 2^-24), t is within 2^-20 of the exact quotient and
// the correctly rounded quotient within 2^-22 of it, so a t farther than
// 2^-19 from every half-integer rounds like the correctly rounded quotient;
// the fast path flags a window of 2^-18 (quant_q's wider one then picks the
// elements it divides). The fast path needs no clamp: every caller's scale is
// the maximum |v| of the values it packs divided by 7, so a finite
// t = v * inv stays within 7 (1 + 2^-22) and rounds to -7..7 (non-finite t
// takes the division). Adding 1.5 * 2^23 to the rounded value puts it, in
// two's complement, in the low bits of the sum, so the code is the sum's low
// nibble; nibble pairs are joined in the low byte of a word and the four
// bytes gathered with two byte permutes.
__device__ __forceinline__ uint32_t pack8(const float v[8], float scale) {
    if (scale == 0.f) return 0;
    const float inv = __fdiv_rn(1.0f, scale);
    bool near = false;
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float t = v[i] * inv;
        const float r = rintf(t);
        near |= !(fabsf(t - r) < 0.5f - 0x1p-18f);
        b[i] = __float_as_uint(r + 0x1.8p23f);
    }
    uint32_t p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = (b[2 * j] & 15u) | (b[2 * j + 1] << 4);
    uint32_t word = __builtin_amdgcn_perm(p[1], p[0], 0x0c0c0400u) |      // bytes 0, 1
                    __builtin_amdgcn_perm(p[3], p[2], 0x04000c0cu);       // bytes 2, 3
    if (near) {
        word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= (uint32_t)(quant_q<-8, 7>(v[i], scale, inv) & 15) << (4 * i);
    }
    return word;
}

// int8: the high-nibble word (q >> 4) and the low-nibble word ((q & 15) - 8)
// of 8 columns.
__device__ __forceinline__ void pack8_w8(const float v[8], float scale, uint32_t& hi, uint32_t& lo) {
    hi = 0;
    lo = 0x88888888u;                       // q = 0 everywhere: h = 0, l = -8
    if (scale == 0.f) return;
    lo = 0;
    const float inv = __fdiv_rn(1.0f, scale);
    bool near = false;
    int q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = quant_fast<-128, 127>(v[i], inv, near);
    if (near) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = quant_q<-128, 127>(v[i], scale, inv);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hi |= (uint32_t)((q[i] >> 4) & 15) << (4 * i);
        lo |= (uint32_t)((q[i] & 15) ^ 8) << (4 * i);
    }
}

// Quantise and store 8 columns c0 .. c0+7 (c0 % 8 == 0) of a row starting at
// qrow: int4 one word at byte c0/2; int8 two words, in the block's high and
// low halves.
template <bool W8>
__device__ __forceinline__ void store8(uint8_t* qrow, int64_t c0, const float v[8], float scale,
                                       int aligned_out) {
    if constexpr (W8) {
        uint32_t hi, lo;
        pack8_w8(v, scale, hi, lo);
        uint8_t* p = qrow + (c0 >> 5) * 32 + ((c0 & 31) >> 1);
        *reinterpret_cast<uint32_t*>(p) = hi;            // int8 rows are 4-byte aligned
        *reinterpret_cast<uint32_t*>(p + 16) = lo;
    } else {
        const uint32_t word = pack8(v, scale);
        uint8_t* p = qrow + c0 / 2;
        if (aligned_out) *reinterpret_cast<uint32_t*>(p) = word;
        else for (int b = 0; b < 4; ++b) p[b] = (uint8_t)(word >> (8 * b));
    }
}

// Value sources of the quantiser: f32 weights, or FP8 e4m3 codes with one f32
// scale per 128 x 128 block (the converter, model card conversion note).
struct F32Src {
    const float* w;
    int64_t cols;
    int aligned;   // 16-byte aligned rows of a multiple of 8 columns
    __device__ __forceinline__ void load8(int64_t r, int64_t c0, float v[8]) const {
        const float* p = w + r * cols + c0;
        if (aligned) {
            const float4 a = *reinterpret_cast<const float4*>(p);
            const float4 b = *reinterpret_cast<const float4*>(p + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = p[i];
        }
    }
    __device__ __forceinline__ float load1(int64_t r, int64_t c) const { return w[r * cols + c]; }
};

// OCP E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa bits,
// subnormals at exponent 0, NaN at S.1111.111, no infinity) are gfx950's FP8
// format: v_cvt_pk_f32_fp8 turns two codes of a word into two exact floats.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float out[4]) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
}

struct Fp8Src {
    const uint8_t* w8;
    const float* sc;   // [ceil(rows/128)][sc_cols]
    int64_t cols, sc_cols;
    int aligned;       // 8-byte aligned rows of a multiple of 8 columns
    __device__ __forceinline__ void load8(int64_t r, int64_t c0, float v[8]) const {
        // 8 columns starting at a multiple of 8 lie in one 128-column block
        const float f = sc[(r >> 7) * sc_cols + (c0 >> 7)];
        const uint8_t* p = w8 + r * cols + c0;
        uint32_t lo, hi;
        if (aligned) {
            const uint2 u = *reinterpret_cast<const uint2*>(p);
            lo = u.x; hi = u.y;
        } else {
            lo = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
            hi = (uint32_t)p[4] | ((uint32_t)p[5] << 8) | ((uint32_t)p[6] << 16) | ((uint32_t)p[7] << 24);
        }
        e4m3x4_to_f32(lo, v);
        e4m3x4_to_f32(hi, v + 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= f;                      // one f32 rounding
    }
    __device__ __forceinline__ float load1(int64_t r, int64_t c) const {
        float x[4];
        e4m3x4_to_f32(w8[r * cols + c], x);
        return x[0] * sc[(r >> 7) * sc_cols + (c >> 7)];
    }
};

// One workgroup per row: block-wide max, then quantise and pack. The first
// NW words of each thread (8 columns each, thread t holding words t + 256 j)
// stay in registers between the max and the packing, so a row of up to
// 2048 NW columns is read once; words beyond are read again (from L2 at best:
// with thousands of rows in flight, a second pass over the whole matrix goes
// back to memory). Loads past the row end are clamped to its last word and
// their values ignored, so every load of the first pass is issued at once.
// One launch covers up to three matrices (an expert's gate, up and down, each
// with its own shape): rows are numbered across them in order, and workgroup
// b takes row b, so the short rows of the last matrix fill the tail of the
// long ones.
template <typename Src>
struct QuantSet {
    Src src[3];
    uint8_t* q[3];
    float* s[3];
    int64_t rows[3];     // 0 for an absent matrix
    int gu_rows[3];      // rows placed at gu_row(r) (an expert's gate or up)
};

template <typename Src, bool W8, int NW>
__global__ __launch_bounds__(256) void quant_row_kernel(QuantSet<Src> mats, int aligned_out) {
    __shared__ float red[4];
    // the matrix of this row (uniform selects: no indexed copy of the argument)
    int64_t r = blockIdx.x;
    int mi = 0;
    if (r >= mats.rows[0]) {
        r -= mats.rows[0];
        mi = 1;
        if (r >= mats.rows[1]) {
            r -= mats.rows[1];
            mi = 2;
        }
    }
    const Src src = mi == 0 ? mats.src[0] : mi == 1 ? mats.src[1] : mats.src[2];
    uint8_t* __restrict__ q = mi == 0 ? mats.q[0] : mi == 1 ? mats.q[1] : mats.q[2];
    float* __restrict__ s = mi == 0 ? mats.s[0] : mi == 1 ? mats.s[1] : mats.s[2];
    const int gu_rows = mi == 0 ? mats.gu_rows[0] : mi == 1 ? mats.gu_rows[1] : mats.gu_rows[2];
    const int64_t cols = src.cols;
    const int64_t words = cols / 8, tail = cols % 8;   // tail is 0, 2, 4 or 6 columns
    float v[NW][8] = {};
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        // register words wholly past a short row's end are not loaded (the
        // condition is the same for the whole workgroup)
        if ((int64_t)j * 256 < words) {
            const int64_t i = threadIdx.x + (int64_t)j * 256;
            src.load8(r, 8 * (i < words ? i : words - 1), v[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < NW; ++j)
        if (threadIdx.x + (int64_t)j * 256 < words)
#pragma unroll
            for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[j][k]));
    for (int64_t i = threadIdx.x + (int64_t)NW * 256; i < words; i += 256) {
        float t[8];
        src.load8(r, 8 * i, t);
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(t[k]));
    }
    if (threadIdx.x == 0)
        for (int64_t c = words * 8; c < cols; ++c) m = fmaxf(m, fabsf(src.load1(r, c)));
    // non-negative and never NaN (fmaxf drops NaN operands): the bits order
    // like the values, so the wave maximum is an integer one over DPP /
    // permlane partners
    m = __uint_as_float(wave_umax(__float_as_uint(m)));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float scale = __fdiv_rn(m, W8 ? 127.0f : 7.0f);
    if (threadIdx.x == 0) s[r] = scale;
    uint8_t* qr = q + (gu_rows ? gu_row(r) : r) * (W8 ? cols : cols / 2);
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int64_t i = threadIdx.x + (int64_t)j * 256;
        if (i < words) store8<W8>(qr, 8 * i, v[j], scale, aligned_out);
    }
    for (int64_t i = threadIdx.x + (int64_t)NW * 256; i < words; i += 256) {
        float t[8];
        src.load8(r, 8 * i, t);
        store8<W8>(qr, 8 * i, t, scale, aligned_out);
    }
    if (!W8 && threadIdx.x == 0 && tail) {           // int8 rows are whole blocks
        float t[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int64_t c = 0; c < tail; ++c) t[c] = src.load1(r, words * 8 + c);
        uint32_t word = pack8(t, scale);
        for (int64_t b = 0; b < tail / 2; ++b) qr[4 * words + b] = (uint8_t)(word >> (8 * b));
    }
}

// gs64: eight threads (lanes 8g..8g+7) per 64-column group.
template <typename Src, bool W8>
__global__ __launch_bounds__(256) void quant_g64_kernel(Src src, int64_t rows, int64_t cols,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ s, int aligned_out,
                                                        int gu_rows) {
    const int64_t words_per_row = cols / 8;
    const int64_t total = rows * words_per_row;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // word index
    // every thread takes part in the shuffles; out-of-range ones carry zeros
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int64_t r = i / words_per_row, wi = i % words_per_row;
    if (i < total) src.load8(r, wi * 8, v);
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    // the group's 8 lanes: DPP partners lane^1, lane^2, lane^7
    m = fmaxf(m, __int_as_float(lane_xchg<1>(__float_as_int(m))));
    m = fmaxf(m, __int_as_float(lane_xchg<2>(__float_as_int(m))));
    m = fmaxf(m, __int_as_float(lane_xchg<4>(__float_as_int(m))));
    const float scale = __fdiv_rn(m, W8 ? 127.0f : 7.0f);
    if (i < total) {
        if ((wi & 7) == 0) s[r * (cols / 64) + wi / 8] = scale;
        store8<W8>(q + (gu_rows ? gu_row(r) : r) * (W8 ? cols : cols / 2), wi * 8, v, scale, aligned_out);
    }
}

// Up to two FP8 matrices of the same shape converted by one launch (an
// expert's gate and up): matrix blockIdx.y.
struct Fp8Pair {
    const uint8_t* w8[2];
    const float* sc[2];
    uint8_t* q[2];
    float* s[2];
};

// FP8 rows of up to 8192 columns, 16-byte aligned, cols % 16 == 0, each
// converted by SPLIT waves of one workgroup (two for rows of 2049 to 6144
// codes, one otherwise). Lane l of wave part p holds units of 16 columns (one
// 16-byte load each) at columns 16 (64 (p NC + c) + l) for c < NC, so every
// load instruction of a wave reads 1 KB of one row; the decoded values stay in
// registers between the row maximum and the packing. gs64: the four lanes of a
// 64-column group share its max through two DPP exchanges.
template <int NC, bool G64, int SPLIT>
__global__ __launch_bounds__(256) void fp8_wave_kernel(Fp8Pair mats, int64_t rows, int64_t cols,
                                                       int64_t sc_cols, int gu_rows) {
    // SPLIT waves of one workgroup share a row: wave part p takes the units
    // [p NC 64, (p + 1) NC 64) and the row maximum is exchanged through LDS
    __shared__ float red[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, part = wave % SPLIT;
    const int64_t r = (int64_t)blockIdx.x * (4 / SPLIT) + wave / SPLIT;
    const bool live = r < rows;                  // the same for the waves of a row
    if (SPLIT == 1 && !live) return;             // whole waves only
    const int mi = blockIdx.y;
    const uint8_t* __restrict__ w8 = mats.w8[mi];
    const float* __restrict__ sc = mats.sc[mi];
    uint8_t* __restrict__ q = mats.q[mi];
    float* __restrict__ s = mats.s[mi];
    const int64_t rr = live ? r : rows - 1;      // dead rows re-read the last one, convert nothing
    uint8_t* qr = q + (gu_rows ? gu_row(rr) : rr) * (cols >> 1);
    const int64_t units = cols >> 4;
    const int64_t ubase = (int64_t)part * NC * 64;
    const uint8_t* row = w8 + rr * cols;
    const float* scr = sc + (rr >> 7) * sc_cols;
    uint4 raw[NC];
    float f[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t u = ubase + (int64_t)c * 64 + lane;
        const int64_t uc = u < units ? u : 0;    // clamped: every load is in bounds
        raw[c] = *reinterpret_cast<const uint4*>(row + uc * 16);
        f[c] = scr[(uc * 16) >> 7];
    }
    float v[NC][16];
    float m = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t u = ubase + (int64_t)c * 64 + lane;
        const bool ok = u < units;
        e4m3x4_to_f32(raw[c].x, &v[c][0]);
        e4m3x4_to_f32(raw[c].y, &v[c][4]);
        e4m3x4_to_f32(raw[c].z, &v[c][8]);
        e4m3x4_to_f32(raw[c].w, &v[c][12]);
        float mc = 0.f;
        if (ubase + (int64_t)(c + 1) * 64 <= units) {   // the whole wave inside the row: no mask
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                v[c][i] *= f[c];
                mc = fmaxf(mc, fabsf(v[c][i]));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                v[c][i] = ok ? v[c][i] * f[c] : 0.f;
                mc = fmaxf(mc, fabsf(v[c][i]));
            }
        }
        if (G64) {
            mc = fmaxf(mc, __int_as_float(lane_xchg<1>(__float_as_int(mc))));
            mc = fmaxf(mc, __int_as_float(lane_xchg<2>(__float_as_int(mc))));
            const float scale = __fdiv_rn(mc, 7.0f);
            if (ok && live) {
                if ((lane & 3) == 0) s[rr * (cols >> 6) + (u >> 2)] = scale;
                uint2 out;
                out.x = pack8(&v[c][0], scale);
                out.y = pack8(&v[c][8], scale);
                *reinterpret_cast<uint2*>(qr + u * 8) = out;
            }
        }
        m = fmaxf(m, mc);
    }
    if (G64) return;
    // the row maximum: m is a non-negative float (never NaN: fmaxf drops NaN
    // operands), so its bits order like its value and the wave's largest is
    // an integer maximum over DPP / permlane partners
    m = __uint_as_float(wave_umax(__float_as_uint(m)));
    if constexpr (SPLIT > 1) {
        if (lane == 0) red[wave] = m;
        __syncthreads();
#pragma unroll
        for (int p = 0; p < SPLIT; ++p) m = fmaxf(m, red[wave - part + p]);
    }
    if (!live) return;
    const float scale = __fdiv_rn(m, 7.0f);
    if (lane == 0 && part == 0) s[rr] = scale;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t u = ubase + (int64_t)c * 64 + lane;
        if (u < units) {
            uint2 out;
            out.x = pack8(&v[c][0], scale);
            out.y = pack8(&v[c][8], scale);
            *reinterpret_cast<uint2*>(qr + u * 8) = out;
        }
    }
}

template <bool G64>
bool launch_fp8_wave(const Fp8Pair& mats, int n_mats, int64_t rows, int64_t cols, int gu_rows,
                     hipStream_t stream) {
    const int64_t nc = (cols / 16 + 63) / 64;
    const int64_t sc_cols = (cols + 127) / 128;
    const dim3 block(256);
    // rows of 3 to 6 units per lane go to two waves each (twice the waves in
    // flight); other widths take one wave per row
    if (nc > 2 && nc <= 6) {
        const dim3 grid((unsigned)((rows + 1) / 2), (unsigned)n_mats);
        if (nc <= 4) launch(fp8_wave_kernel<2, G64, 2>, grid, block, 0, stream, mats, rows, cols, sc_cols, gu_rows);
        else launch(fp8_wave_kernel<3, G64, 2>, grid, block, 0, stream, mats, rows, cols, sc_cols, gu_rows);
        return true;
    }
    const dim3 grid((unsigned)((rows + 3) / 4), (unsigned)n_mats);
    if (nc <= 1) launch(fp8_wave_kernel<1, G64, 1>, grid, block, 0, stream, mats, rows, cols, sc_cols, gu_rows);
    else if (nc <= 2) launch(fp8_wave_kernel<2, G64, 1>, grid, block, 0, stream, mats, rows, cols, sc_cols, gu_rows);
    else if (nc <= 8) launch(fp8_wave_kernel<8, G64, 1>, grid, block, 0, stream, mats, rows, cols, sc_cols, gu_rows);
    else return false;
    return true;
}

// The one-wave-per-row kernel takes rows of 16-byte aligned codes, whole
// 16-column units, at most 8192 columns, and 8-byte aligned int4 rows.
bool fp8_wave_fits(const uint8_t* w8, const uint8_t* q, int64_t rows, int64_t cols,
                   int32_t wbits) {
    return wbits != 8 && (uintptr_t)w8 % 16 == 0 && (uintptr_t)q % 8 == 0 && cols % 16 == 0 &&
           cols <= 8192 && rows <= 0x1fffffffLL;
}

// Per-row scales for the matrices of a set in one launch; max_cols is the
// widest row (it sets the words each thread keeps in registers).
template <typename Src, bool W8>
coli_status launch_quant_set(const QuantSet<Src>& mats, int64_t max_cols, int aligned_out,
                             hipStream_t stream) {
    const int64_t total = mats.rows[0] + mats.rows[1] + mats.rows[2];
    if (total > 0x7fffffffLL) return fail(COLI_EUNSUPPORTED, "quantize: too many rows");
    if (total == 0) return COLI_OK;
    // words of 8 columns per thread kept in registers: the widest row's, up to 4
    const int64_t nw = (max_cols / 8 + 255) / 256;
    const dim3 grid((unsigned)total), block(256);
    if (nw <= 1) launch(quant_row_kernel<Src, W8, 1>, grid, block, 0, stream, mats, aligned_out);
    else if (nw <= 2) launch(quant_row_kernel<Src, W8, 2>, grid, block, 0, stream, mats, aligned_out);
    else if (nw <= 3) launch(quant_row_kernel<Src, W8, 3>, grid, block, 0, stream, mats, aligned_out);
    else launch(quant_row_kernel<Src, W8, 4>, grid, block, 0, stream, mats, aligned_out);
    return COLI_OK;
}

// Per-row scales: one launch for matrix a, or for a and the same-shaped b
// (b_src non-null; same aligned_out). gs64: matrix a only.
template <typename Src, bool W8>
coli_status launch_quant_t(const Src& src, int64_t rows, int64_t cols, int32_t group, uint8_t* q,
                           float* s, int aligned_out, int gu_rows, hipStream_t stream,
                           const Src* b_src = nullptr, uint8_t* b_q = nullptr,
                           float* b_s = nullptr) {
    if (group == 0) {
        if (rows > 0x7fffffffLL) return fail(COLI_EUNSUPPORTED, "quantize: too many rows");
        QuantSet<Src> mats{};
        mats.src[0] = mats.src[1] = mats.src[2] = src;
        mats.q[0] = mats.q[1] = mats.q[2] = q;
        mats.s[0] = mats.s[1] = mats.s[2] = s;
        mats.rows[0] = rows;
        mats.gu_rows[0] = mats.gu_rows[1] = gu_rows;
        if (b_src) {
            mats.src[1] = *b_src;
            mats.q[1] = b_q;
            mats.s[1] = b_s;
            mats.rows[1] = rows;
        }
        return launch_quant_set<Src, W8>(mats, cols, aligned_out, stream);
    } else {
        // the group of 8 lanes must not straddle rows: cols % 64 == 0 is required
        const int64_t total = rows * (cols / 8);
        const int64_t blocks = (total + 255) / 256;
        if (blocks > 0x7fffffffLL) return fail(COLI_EUNSUPPORTED, "quantize: tensor too large");
        launch(quant_g64_kernel<Src, W8>, dim3((unsigned)blocks), dim3(256), 0, stream, src, rows,
               cols, q, s, aligned_out, gu_rows);
    }
    return COLI_OK;
}

template <typename Src>
coli_status launch_quant(const Src& src, int64_t rows, int64_t cols, int32_t group, uint8_t* q,
                         float* s, int aligned_out, hipStream_t stream, int32_t wbits, int gu_rows,
                         const Src* b_src = nullptr, uint8_t* b_q = nullptr, float* b_s = nullptr) {
    if (rows == 0) return COLI_OK;
    coli_status st;
    if (wbits == 8) {
        if (cols % kBlock || (uintptr_t)q % 4 || (b_src && (uintptr_t)b_q % 4))
            return fail(COLI_EINVAL, "quantize: int8 rows need cols % 32 == 0 and 4-byte alignment");
        st = launch_quant_t<Src, true>(src, rows, cols, group, q, s, 1, gu_rows, stream, b_src, b_q, b_s);
    } else {
        st = launch_quant_t<Src, false>(src, rows, cols, group, q, s, aligned_out, gu_rows, stream,
                                        b_src, b_q, b_s);
    }
    if (st) return st;
    COLI_CHECK_LAUNCH("quantize kernel launch");
    return COLI_OK;
}

}  // namespace

coli_status launch_quantize(const float* w, int64_t rows, int64_t cols, int32_t group, uint8_t* q,
                            float* s, hipStream_t stream, int32_t wbits, bool gu_rows) {
    const int aligned = ((uintptr_t)w % 16 == 0) && ((uintptr_t)q % 4 == 0) &&
                        (cols % 8 == 0) ? 1 : 0;
    F32Src src{w, cols, aligned};
    return launch_quant(src, rows, cols, group, q, s, aligned, stream, wbits, gu_rows ? 1 : 0);
}

coli_status launch_quantize_pair(const float* wa, uint8_t* qa, float* sa, const float* wb,
                                 uint8_t* qb, float* sb, int64_t rows, int64_t cols,
                                 int32_t group, hipStream_t stream, int32_t wbits, bool gu_rows) {
    const int al_a = ((uintptr_t)wa % 16 == 0) && ((uintptr_t)qa % 4 == 0) && (cols % 8 == 0) ? 1 : 0;
    const int al_b = ((uintptr_t)wb % 16 == 0) && ((uintptr_t)qb % 4 == 0) && (cols % 8 == 0) ? 1 : 0;
    if (group != 0 || al_a != al_b) {
        coli_status st = launch_quantize(wa, rows, cols, group, qa, sa, stream, wbits, gu_rows);
        if (st) return st;
        return launch_quantize(wb, rows, cols, group, qb, sb, stream, wbits, gu_rows);
    }
    const F32Src a{wa, cols, al_a}, b{wb, cols, al_b};
    return launch_quant(a, rows, cols, group, qa, sa, al_a, stream, wbits, gu_rows ? 1 : 0, &b, qb, sb);
}

coli_status launch_quantize_expert(const float* wg, uint8_t* qg, float* sg, const float* wu,
                                   uint8_t* qu, float* su, const float* wd, uint8_t* qd, float* sd,
                                   int64_t H, int64_t I, int32_t group, hipStream_t stream,
                                   int32_t wbits) {
    auto al = [](const float* w, const uint8_t* q, int64_t cols) {
        return ((uintptr_t)w % 16 == 0) && ((uintptr_t)q % 4 == 0) && (cols % 8 == 0) ? 1 : 0;
    };
    const int ag = al(wg, qg, H), au = al(wu, qu, H), ad = al(wd, qd, I);
    const bool w8_ok = wbits != 8 || (H % kBlock == 0 && I % kBlock == 0 && (uintptr_t)qg % 4 == 0 &&
                                      (uintptr_t)qu % 4 == 0 && (uintptr_t)qd % 4 == 0);
    if (group != 0 || ag != au || ag != ad || !w8_ok || I == 0 || H == 0) {
        coli_status st = launch_quantize_pair(wg, qg, sg, wu, qu, su, I, H, group, stream, wbits, true);
        if (st) return st;
        return launch_quantize(wd, H, I, group, qd, sd, stream, wbits, false);
    }
    QuantSet<F32Src> mats{};
    mats.src[0] = F32Src{wg, H, ag};
    mats.src[1] = F32Src{wu, H, au};
    mats.src[2] = F32Src{wd, I, ad};
    mats.q[0] = qg;
    mats.q[1] = qu;
    mats.q[2] = qd;
    mats.s[0] = sg;
    mats.s[1] = su;
    mats.s[2] = sd;
    mats.rows[0] = mats.rows[1] = I;
    mats.rows[2] = H;
    mats.gu_rows[0] = mats.gu_rows[1] = 1;
    const int64_t wide = H > I ? H : I;
    const coli_status st = wbits == 8 ? launch_quant_set<F32Src, true>(mats, wide, 1, stream)
                                      : launch_quant_set<F32Src, false>(mats, wide, ag, stream);
    if (st) return st;
    COLI_CHECK_LAUNCH("quantize kernel launch");
    return COLI_OK;
}

coli_status launch_convert_fp8(const uint8_t* w8, const float* scale, int64_t rows, int64_t cols,
                               int32_t group, uint8_t* q, float* s, hipStream_t stream,
                               int32_t wbits, bool gu_rows) {
    if (rows == 0) return COLI_OK;
    if (fp8_wave_fits(w8, q, rows, cols, wbits)) {
        const Fp8Pair one{{w8, w8}, {scale, scale}, {q, q}, {s, s}};
        const bool ok = group == 0 ? launch_fp8_wave<false>(one, 1, rows, cols, gu_rows ? 1 : 0, stream)
                                   : launch_fp8_wave<true>(one, 1, rows, cols, gu_rows ? 1 : 0, stream);
        if (ok) {
            COLI_CHECK_LAUNCH("fp8 convert kernel launch");
            return COLI_OK;
        }
    }
    const int aligned_in = ((uintptr_t)w8 % 8 == 0) && (cols % 8 == 0) ? 1 : 0;
    const int aligned_out = ((uintptr_t)q % 4 == 0) && (cols % 8 == 0) ? 1 : 0;
    Fp8Src src{w8, scale, cols, (cols + 127) / 128, aligned_in};
    return launch_quant(src, rows, cols, group, q, s, aligned_out, stream, wbits, gu_rows ? 1 : 0);
}

coli_status launch_convert_fp8_pair(const uint8_t* w8a, const float* scale_a, uint8_t* qa,
                                    float* sa, const uint8_t* w8b, const float* scale_b,
                                    uint8_t* qb, float* sb, int64_t rows, int64_t cols,
                                    int32_t group, hipStream_t stream, int32_t wbits,
                                    bool gu_rows) {
    if (rows == 0) return COLI_OK;
    if (fp8_wave_fits(w8a, qa, rows, cols, wbits) && fp8_wave_fits(w8b, qb, rows, cols, wbits)) {
        const Fp8Pair two{{w8a, w8b}, {scale_a, scale_b}, {qa, qb}, {sa, sb}};
        const bool ok = group == 0 ? launch_fp8_wave<false>(two, 2, rows, cols, gu_rows ? 1 : 0, stream)
                                   : launch_fp8_wave<true>(two, 2, rows, cols, gu_rows ? 1 : 0, stream);
        if (ok) {
            COLI_CHECK_LAUNCH("fp8 convert kernel launch");
            return COLI_OK;
        }
    }
    coli_status st = launch_convert_fp8(w8a, scale_a, rows, cols, group, qa, sa, stream, wbits, gu_rows);
    if (st) return st;
    return launch_convert_fp8(w8b, scale_b, rows, cols, group, qb, sb, stream, wbits, gu_rows);
}

}  // namespace coli
