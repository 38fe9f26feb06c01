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

namespace coli {
namespace {

// q = rint(v / scale) with IEEE division, clamped to [QLO, QHI]. The quotient
// is first formed as v * inv with inv = 1/scale correctly rounded: |q| <= 128
// keeps that within 2^-15 of the correctly rounded quotient, so the two can
// round to different integers only when t lies within 2^-15 of a
// half-integer. Such values (and non-finite t, e.g. from a subnormal scale)
// take the division.
template <int QLO, int QHI>
__device__ __forceinline__ int quant_q(float v, float scale, float inv) {
    const float t = v * inv;
    float r = rintf(t);
    if (!(fabsf(fabsf(t - r) - 0.5f) > 0x1p-14f)) r = rintf(__fdiv_rn(v, scale));
    return (int)fminf(fmaxf(r, (float)QLO), (float)QHI);
}

// int4: 8 nibbles of one output word.
__device__ __forceinline__ uint32_t pack8(const float v[8], float scale) {
    uint32_t word = 0;
    if (scale == 0.f) return 0;
    const float inv = __fdiv_rn(1.0f, scale);
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= (uint32_t)(quant_q<-8, 7>(v[i], scale, inv) & 15) << (4 * i);
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
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int q = quant_q<-128, 127>(v[i], scale, inv);
        hi |= (uint32_t)((q >> 4) & 15) << (4 * i);
        lo |= (uint32_t)((q & 15) ^ 8) << (4 * i);
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

// One workgroup per row: block-wide max, then quantise and pack.
template <typename Src, bool W8>
__global__ __launch_bounds__(256) void quant_row_kernel(Src src, int64_t cols,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ s, int aligned_out) {
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const int64_t words = cols / 8, tail = cols % 8;   // tail is 0, 2, 4 or 6 columns
    float m = 0.f;
    for (int64_t i = threadIdx.x; i < words; i += blockDim.x) {
        float v[8];
        src.load8(r, 8 * i, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    }
    if (threadIdx.x == 0)
        for (int64_t c = words * 8; c < cols; ++c) m = fmaxf(m, fabsf(src.load1(r, c)));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float scale = __fdiv_rn(m, W8 ? 127.0f : 7.0f);
    if (threadIdx.x == 0) s[r] = scale;
    uint8_t* qr = q + r * (W8 ? cols : cols / 2);
    for (int64_t i = threadIdx.x; i < words; i += blockDim.x) {
        float v[8];
        src.load8(r, 8 * i, v);
        store8<W8>(qr, 8 * i, v, scale, aligned_out);
    }
    if (!W8 && threadIdx.x == 0 && tail) {           // int8 rows are whole blocks
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int64_t c = 0; c < tail; ++c) v[c] = src.load1(r, words * 8 + c);
        uint32_t word = pack8(v, scale);
        for (int64_t b = 0; b < tail / 2; ++b) qr[4 * words + b] = (uint8_t)(word >> (8 * b));
    }
}

// gs64: eight threads (lanes 8g..8g+7) per 64-column group.
template <typename Src, bool W8>
__global__ __launch_bounds__(256) void quant_g64_kernel(Src src, int64_t rows, int64_t cols,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ s, int aligned_out) {
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
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    const float scale = __fdiv_rn(m, W8 ? 127.0f : 7.0f);
    if (i < total) {
        if ((wi & 7) == 0) s[r * (cols / 64) + wi / 8] = scale;
        store8<W8>(q + r * (W8 ? cols : cols / 2), wi * 8, v, scale, aligned_out);
    }
}

// FP8 rows of up to 8192 columns, 16-byte aligned, cols % 16 == 0: one wave
// per row. Lane l holds units of 16 columns (one 16-byte load each) at
// columns 16 (64 c + l) for c < NC, so every load instruction of the wave
// reads 1 KB of one row; the decoded row stays in registers between the max
// and the packing. gs64: the four lanes of a 64-column group share its max
// through two shuffles.
template <int NC, bool G64>
__global__ __launch_bounds__(256) void fp8_wave_kernel(const uint8_t* __restrict__ w8,
                                                       const float* __restrict__ sc,
                                                       int64_t rows, int64_t cols,
                                                       int64_t sc_cols, uint8_t* __restrict__ q,
                                                       float* __restrict__ s) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;                       // whole waves only
    const int64_t units = cols >> 4;
    const uint8_t* row = w8 + r * cols;
    const float* scr = sc + (r >> 7) * sc_cols;
    uint4 raw[NC];
    float f[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t u = (int64_t)c * 64 + lane;
        const int64_t uc = u < units ? u : 0;    // clamped: every load is in bounds
        raw[c] = *reinterpret_cast<const uint4*>(row + uc * 16);
        f[c] = scr[(uc * 16) >> 7];
    }
    float v[NC][16];
    float m = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const bool ok = (int64_t)c * 64 + lane < units;
        e4m3x4_to_f32(raw[c].x, &v[c][0]);
        e4m3x4_to_f32(raw[c].y, &v[c][4]);
        e4m3x4_to_f32(raw[c].z, &v[c][8]);
        e4m3x4_to_f32(raw[c].w, &v[c][12]);
        float mc = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            v[c][i] = ok ? v[c][i] * f[c] : 0.f;
            mc = fmaxf(mc, fabsf(v[c][i]));
        }
        if (G64) {
            mc = fmaxf(mc, __shfl_xor(mc, 1));
            mc = fmaxf(mc, __shfl_xor(mc, 2));
            const float scale = __fdiv_rn(mc, 7.0f);
            if (ok) {
                const int64_t u = (int64_t)c * 64 + lane;
                if ((lane & 3) == 0) s[r * (cols >> 6) + (u >> 2)] = scale;
                uint2 out;
                out.x = pack8(&v[c][0], scale);
                out.y = pack8(&v[c][8], scale);
                *reinterpret_cast<uint2*>(q + r * (cols >> 1) + u * 8) = out;
            }
        }
        m = fmaxf(m, mc);
    }
    if (G64) return;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float scale = __fdiv_rn(m, 7.0f);
    if (lane == 0) s[r] = scale;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t u = (int64_t)c * 64 + lane;
        if (u < units) {
            uint2 out;
            out.x = pack8(&v[c][0], scale);
            out.y = pack8(&v[c][8], scale);
            *reinterpret_cast<uint2*>(q + r * (cols >> 1) + u * 8) = out;
        }
    }
}

template <bool G64>
bool launch_fp8_wave(const uint8_t* w8, const float* scale, int64_t rows, int64_t cols,
                     uint8_t* q, float* s, hipStream_t stream) {
    const int64_t nc = (cols / 16 + 63) / 64;
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    const int64_t sc_cols = (cols + 127) / 128;
    if (nc <= 1) launch(fp8_wave_kernel<1, G64>, grid, block, 0, stream, w8, scale, rows, cols, sc_cols, q, s);
    else if (nc <= 2) launch(fp8_wave_kernel<2, G64>, grid, block, 0, stream, w8, scale, rows, cols, sc_cols, q, s);
    else if (nc <= 4) launch(fp8_wave_kernel<4, G64>, grid, block, 0, stream, w8, scale, rows, cols, sc_cols, q, s);
    else if (nc <= 6) launch(fp8_wave_kernel<6, G64>, grid, block, 0, stream, w8, scale, rows, cols, sc_cols, q, s);
    else if (nc <= 8) launch(fp8_wave_kernel<8, G64>, grid, block, 0, stream, w8, scale, rows, cols, sc_cols, q, s);
    else return false;
    return true;
}

template <typename Src, bool W8>
coli_status launch_quant_t(const Src& src, int64_t rows, int64_t cols, int32_t group, uint8_t* q,
                           float* s, int aligned_out, hipStream_t stream) {
    if (group == 0) {
        if (rows > 0x7fffffffLL) return fail(COLI_EUNSUPPORTED, "quantize: too many rows");
        launch(quant_row_kernel<Src, W8>, dim3((unsigned)rows), dim3(256), 0, stream, src,
               cols, q, s, aligned_out);
    } else {
        // the group of 8 lanes must not straddle rows: cols % 64 == 0 is required
        const int64_t total = rows * (cols / 8);
        const int64_t blocks = (total + 255) / 256;
        if (blocks > 0x7fffffffLL) return fail(COLI_EUNSUPPORTED, "quantize: tensor too large");
        launch(quant_g64_kernel<Src, W8>, dim3((unsigned)blocks), dim3(256), 0, stream, src, rows,
               cols, q, s, aligned_out);
    }
    return COLI_OK;
}

template <typename Src>
coli_status launch_quant(const Src& src, int64_t rows, int64_t cols, int32_t group, uint8_t* q,
                         float* s, int aligned_out, hipStream_t stream, int32_t wbits) {
    if (rows == 0) return COLI_OK;
    coli_status st;
    if (wbits == 8) {
        if (cols % kBlock || (uintptr_t)q % 4)
            return fail(COLI_EINVAL, "quantize: int8 rows need cols % 32 == 0 and 4-byte alignment");
        st = launch_quant_t<Src, true>(src, rows, cols, group, q, s, 1, stream);
    } else {
        st = launch_quant_t<Src, false>(src, rows, cols, group, q, s, aligned_out, stream);
    }
    if (st) return st;
    COLI_CHECK_LAUNCH("quantize kernel launch");
    return COLI_OK;
}

}  // namespace

coli_status launch_quantize(const float* w, int64_t rows, int64_t cols, int32_t group, uint8_t* q,
                            float* s, hipStream_t stream, int32_t wbits) {
    const int aligned = ((uintptr_t)w % 16 == 0) && ((uintptr_t)q % 4 == 0) &&
                        (cols % 8 == 0) ? 1 : 0;
    F32Src src{w, cols, aligned};
    return launch_quant(src, rows, cols, group, q, s, aligned, stream, wbits);
}

coli_status launch_convert_fp8(const uint8_t* w8, const float* scale, int64_t rows, int64_t cols,
                               int32_t group, uint8_t* q, float* s, hipStream_t stream,
                               int32_t wbits) {
    if (rows == 0) return COLI_OK;
    if (wbits != 8 && (uintptr_t)w8 % 16 == 0 && (uintptr_t)q % 8 == 0 && cols % 16 == 0 &&
        cols <= 8192 && rows <= 0x1fffffffLL) {
        const bool ok = group == 0 ? launch_fp8_wave<false>(w8, scale, rows, cols, q, s, stream)
                                   : launch_fp8_wave<true>(w8, scale, rows, cols, q, s, stream);
        if (ok) {
            COLI_CHECK_LAUNCH("fp8 convert kernel launch");
            return COLI_OK;
        }
    }
    const int aligned_in = ((uintptr_t)w8 % 8 == 0) && (cols % 8 == 0) ? 1 : 0;
    const int aligned_out = ((uintptr_t)q % 4 == 0) && (cols % 8 == 0) ? 1 : 0;
    Fp8Src src{w8, scale, cols, (cols + 127) / 128, aligned_in};
    return launch_quant(src, rows, cols, group, q, s, aligned_out, stream, wbits);
}

}  // namespace coli
