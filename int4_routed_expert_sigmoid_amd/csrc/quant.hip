// int4 quantiser (the container rule of the model card "jlnsrk/GLM-5.2-colibri-int4":
// packed int4 nibbles + F32 scales, values rounded half-to-even as np.rint /
// lrintf do; gs64 group scales from the practical guide's section 三).
//
// scale = max|w| / 7 (float division) per row or per 64 consecutive columns,
// q = rint(w / scale) (float division, nearest-even), clamped to [-8, 7];
// scale 0 gives q = 0. Each thread owns 8 consecutive columns, i.e. one
// 32-bit word of packed output.
#include "common.h"

namespace coli {
namespace {

__device__ __forceinline__ uint32_t pack8(const float v[8], float scale) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int q = 0;
        if (scale != 0.f) {
            float r = rintf(__fdiv_rn(v[i], scale));
            r = fminf(fmaxf(r, -8.f), 7.f);
            q = (int)r;
        }
        word |= (uint32_t)(q & 15) << (4 * i);
    }
    return word;
}

__device__ __forceinline__ void load8(const float* p, float v[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8_unaligned(const float* p, float v[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[i];
}

// One workgroup per row: block-wide max, then quantise and pack.
__global__ __launch_bounds__(256) void quant_row_kernel(const float* __restrict__ w, int64_t rows,
                                                        int64_t cols, uint8_t* __restrict__ q,
                                                        float* __restrict__ s, int aligned) {
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const float* wr = w + r * cols;
    const int64_t words = cols / 8, tail = cols % 8;   // tail is 0, 2, 4 or 6 columns
    float m = 0.f;
    for (int64_t i = threadIdx.x; i < words; i += blockDim.x) {
        float v[8];
        if (aligned) load8(wr + 8 * i, v); else load8_unaligned(wr + 8 * i, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    }
    if (threadIdx.x == 0)
        for (int64_t c = words * 8; c < cols; ++c) m = fmaxf(m, fabsf(wr[c]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float scale = __fdiv_rn(m, 7.0f);
    if (threadIdx.x == 0) s[r] = scale;
    uint8_t* qr = q + r * (cols / 2);
    for (int64_t i = threadIdx.x; i < words; i += blockDim.x) {
        float v[8];
        if (aligned) load8(wr + 8 * i, v); else load8_unaligned(wr + 8 * i, v);
        uint32_t word = pack8(v, scale);
        if (aligned) *reinterpret_cast<uint32_t*>(qr + 4 * i) = word;
        else for (int b = 0; b < 4; ++b) qr[4 * i + b] = (uint8_t)(word >> (8 * b));
    }
    if (threadIdx.x == 0 && tail) {
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int64_t c = 0; c < tail; ++c) v[c] = wr[words * 8 + c];
        uint32_t word = pack8(v, scale);
        for (int64_t b = 0; b < tail / 2; ++b) qr[4 * words + b] = (uint8_t)(word >> (8 * b));
    }
}

// gs64: eight threads (lanes 8g..8g+7) per 64-column group.
__global__ __launch_bounds__(256) void quant_g64_kernel(const float* __restrict__ w, int64_t rows,
                                                        int64_t cols, uint8_t* __restrict__ q,
                                                        float* __restrict__ s, int aligned) {
    const int64_t words_per_row = cols / 8;
    const int64_t total = rows * words_per_row;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // word index
    // every thread takes part in the shuffles; out-of-range ones carry zeros
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int64_t r = i / words_per_row, wi = i % words_per_row;
    if (i < total) {
        const float* p = w + r * cols + wi * 8;
        if (aligned) load8(p, v); else load8_unaligned(p, v);
    }
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    const float scale = __fdiv_rn(m, 7.0f);
    if (i < total) {
        if ((wi & 7) == 0) s[r * (cols / 64) + wi / 8] = scale;
        uint32_t word = pack8(v, scale);
        uint8_t* qp = q + r * (cols / 2) + wi * 4;
        if (aligned) *reinterpret_cast<uint32_t*>(qp) = word;
        else for (int b = 0; b < 4; ++b) qp[b] = (uint8_t)(word >> (8 * b));
    }
}

}  // namespace

coli_status launch_quantize(const float* w, int64_t rows, int64_t cols, int32_t group, uint8_t* q,
                            float* s, hipStream_t stream) {
    if (rows == 0) return COLI_OK;
    const int aligned = ((uintptr_t)w % 16 == 0) && ((uintptr_t)q % 4 == 0) &&
                        (cols % 8 == 0) ? 1 : 0;
    if (group == 0) {
        if (rows > 0x7fffffffLL) return fail(COLI_EUNSUPPORTED, "quantize: too many rows");
        launch(quant_row_kernel, dim3((unsigned)rows), dim3(256), 0, stream, w, rows,
                           cols, q, s, aligned);
    } else {
        // the group of 8 lanes must not straddle rows: cols % 64 == 0 is required
        const int64_t total = rows * (cols / 8);
        const int64_t blocks = (total + 255) / 256;
        if (blocks > 0x7fffffffLL) return fail(COLI_EUNSUPPORTED, "quantize: tensor too large");
        launch(quant_g64_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, rows,
                           cols, q, s, aligned);
    }
    COLI_CHECK_LAUNCH("quantize kernel launch");
    return COLI_OK;
}

}  // namespace coli
