// int4 dequant GEMV family for decode and small per-expert token counts.
//
// Expert FFN (practical guide section 二: gate, up and down stored adjacently;
// SwiGLU): h = silu(gate x) * (up x), y = down h, for every (expert, token)
// pair of a work list, each expert's weights streamed once per pass of up to
// MT tokens.
//
// Layout of the work: a workgroup takes 32 rows of one expert's gate and up
// matrices (or 64 rows of its down matrix). Every thread owns fixed 32-column
// blocks of the reduction axis, loads the 16 bytes (32 nibbles) of each row
// that fall in its blocks with one 128-bit load, and multiplies them by the
// activation's digit planes (common.h) with v_dot8_i32_i4: the per-block sum
// sum_c q_c X_c is exact in int32 and is scaled once (block scale x row or
// group scale) into an f32 partial. Partials are reduced across the wave and,
// for gate/up rows wider than one wave, across waves through LDS. gate/up
// workgroups finish by applying SiLU, multiplying, and encoding their 32
// h values as one digit block for the down pass.
#include "common.h"
#include "profile.h"

namespace coli {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming 128-bit load of weight nibbles (read once: non-temporal).
__device__ __forceinline__ uint4 ldg128(const uint8_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// x [rows][K] f32 -> planes [rows][K/32][5][4] u32, scales [rows][K/32].
__global__ __launch_bounds__(256) void encode_kernel(const float* __restrict__ x, int rows, int K,
                                                     uint32_t* __restrict__ planes,
                                                     float* __restrict__ scales) {
    const int C = K / kBlock;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int q = (int)(gid & 3);
    const int64_t blk = gid >> 2;
    const int64_t row = blk / C;
    const int b = (int)(blk % C);
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const bool ok = row < rows;
    if (ok) {
        const float* p = x + row * K + b * kBlock + q * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = p[i];
    }
    uint32_t words[kPlanes];
    const float sc = encode_quarter(v, words);
    if (ok) {
        uint32_t* out = planes + (row * C + b) * kWordsPerBlock;
#pragma unroll
        for (int p = 0; p < kPlanes; ++p) out[p * 4 + q] = words[p];
        if (q == 0) scales[row * C + b] = sc;
    }
}

// ----------------------------------------------------------------- gate/up
template <int W, int NCH, int MT, bool GS>
__global__ __launch_bounds__(64 * W) void gateup_kernel(
    const WorkItem* __restrict__ items, const int32_t* __restrict__ n_items,
    const int32_t* __restrict__ rows_tok, const int32_t* __restrict__ rows_out,
    const uint32_t* __restrict__ xplanes, const float* __restrict__ xscale,
    uint32_t* __restrict__ hplanes, float* __restrict__ hscale, int H, int I, BlobLayout L) {
    const int item = blockIdx.y;
    if (item >= *n_items) return;
    const WorkItem it = items[item];
    const int tile = blockIdx.x;
    const int r0 = tile * kBlock;
    const int C = H / kBlock, CI = I / kBlock;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint8_t* gq = it.blob + L.gate_q;
    const uint8_t* uq = it.blob + L.up_q;
    const float* gsc = reinterpret_cast<const float*>(it.blob + L.gate_s);
    const float* usc = reinterpret_cast<const float*>(it.blob + L.up_s);
    const size_t rowbytes = (size_t)H / 2;
    const int gpr = GS ? H / 64 : 1;

    __shared__ float red[W][kBlock][MT][2];
    __shared__ float hval[MT][kBlock];

    for (int m0 = 0; m0 < it.count; m0 += MT) {
        const int mc = min(MT, it.count - m0);
        uint4 xp[MT][NCH][kPlanes];
        float xs[MT][NCH];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int tok = (m < mc) ? rows_tok[it.begin + m0 + m] : 0;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int ch = tid + 64 * W * j;
                if (m < mc && ch < C) {
                    const uint4* src = reinterpret_cast<const uint4*>(
                        xplanes + ((size_t)tok * C + ch) * kWordsPerBlock);
#pragma unroll
                    for (int p = 0; p < kPlanes; ++p) xp[m][j][p] = src[p];
                    xs[m][j] = xscale[(size_t)tok * C + ch];
                } else {
#pragma unroll
                    for (int p = 0; p < kPlanes; ++p) xp[m][j][p] = make_uint4(0, 0, 0, 0);
                    xs[m][j] = 0.f;
                }
            }
        }
#pragma unroll 2
        for (int r = 0; r < kBlock; ++r) {
            const int row = r0 + r;
            float pg[MT], pu[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) { pg[m] = 0.f; pu[m] = 0.f; }
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int ch = tid + 64 * W * j;
                if (ch < C) {
                    const uint4 wg = ldg128(gq + row * rowbytes + (size_t)ch * 16);
                    const uint4 wu = ldg128(uq + row * rowbytes + (size_t)ch * 16);
                    float fg = 1.f, fu = 1.f;
                    if (GS) {
                        fg = gsc[(size_t)row * gpr + (ch >> 1)];
                        fu = usc[(size_t)row * gpr + (ch >> 1)];
                    }
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        if (m < mc) {
                            pg[m] += (float)block_dot(wg, xp[m][j]) * (xs[m][j] * fg);
                            pu[m] += (float)block_dot(wu, xp[m][j]) * (xs[m][j] * fu);
                        }
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m < mc) {
                    const float g = wave_sum(pg[m]);
                    const float u = wave_sum(pu[m]);
                    if (lane == 0) { red[wave][r][m][0] = g; red[wave][r][m][1] = u; }
                }
            }
        }
        __syncthreads();
        for (int i = tid; i < kBlock * MT; i += 64 * W) {
            const int r = i & (kBlock - 1), m = i / kBlock;
            if (m < mc) {
                float g = 0.f, u = 0.f;
#pragma unroll
                for (int w = 0; w < W; ++w) { g += red[w][r][m][0]; u += red[w][r][m][1]; }
                if (!GS) { g *= gsc[r0 + r]; u *= usc[r0 + r]; }
                hval[m][r] = g / (1.f + expf(-g)) * u;
            }
        }
        __syncthreads();
        if (tid < 4 * MT) {
            const int m = tid >> 2, q = tid & 3;
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = (m < mc) ? hval[m][q * 8 + i] : 0.f;
            uint32_t words[kPlanes];
            const float sc = encode_quarter(v, words);
            if (m < mc) {
                const int out = rows_out[it.begin + m0 + m];
                uint32_t* dst = hplanes + ((size_t)out * CI + tile) * kWordsPerBlock;
#pragma unroll
                for (int p = 0; p < kPlanes; ++p) dst[p * 4 + q] = words[p];
                if (q == 0) hscale[(size_t)out * CI + tile] = sc;
            }
        }
        __syncthreads();
    }
}

// -------------------------------------------------------------------- down
constexpr int kDownRowsPerWave = 16;
constexpr int kDownRowsPerBlock = 4 * kDownRowsPerWave;

template <int NCH, int MT, bool GS>
__global__ __launch_bounds__(256) void down_kernel(
    const WorkItem* __restrict__ items, const int32_t* __restrict__ n_items,
    const int32_t* __restrict__ rows_out, const uint32_t* __restrict__ hplanes,
    const float* __restrict__ hscale, float* __restrict__ y_rows, int H, int I, BlobLayout L) {
    const int item = blockIdx.y;
    if (item >= *n_items) return;
    const WorkItem it = items[item];
    const int CI = I / kBlock;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rbase = blockIdx.x * kDownRowsPerBlock + wave * kDownRowsPerWave;
    const uint8_t* dq = it.blob + L.down_q;
    const float* dsc = reinterpret_cast<const float*>(it.blob + L.down_s);
    const size_t rowbytes = (size_t)I / 2;
    const int gpr = GS ? I / 64 : 1;

    for (int m0 = 0; m0 < it.count; m0 += MT) {
        const int mc = min(MT, it.count - m0);
        uint4 hp[MT][NCH][kPlanes];
        float hs[MT][NCH];
        int outr[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            outr[m] = (m < mc) ? rows_out[it.begin + m0 + m] : 0;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int ch = lane + 64 * j;
                if (m < mc && ch < CI) {
                    const uint4* src = reinterpret_cast<const uint4*>(
                        hplanes + ((size_t)outr[m] * CI + ch) * kWordsPerBlock);
#pragma unroll
                    for (int p = 0; p < kPlanes; ++p) hp[m][j][p] = src[p];
                    hs[m][j] = hscale[(size_t)outr[m] * CI + ch];
                } else {
#pragma unroll
                    for (int p = 0; p < kPlanes; ++p) hp[m][j][p] = make_uint4(0, 0, 0, 0);
                    hs[m][j] = 0.f;
                }
            }
        }
#pragma unroll 2
        for (int r = 0; r < kDownRowsPerWave; ++r) {
            const int row = rbase + r;
            if (row >= H) break;
            float acc[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = 0.f;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int ch = lane + 64 * j;
                if (ch < CI) {
                    const uint4 w = ldg128(dq + row * rowbytes + (size_t)ch * 16);
                    const float f = GS ? dsc[(size_t)row * gpr + (ch >> 1)] : 1.f;
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        if (m < mc) acc[m] += (float)block_dot(w, hp[m][j]) * (hs[m][j] * f);
                }
            }
            const float rs = GS ? 1.f : dsc[row];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m < mc) {
                    const float v = wave_sum(acc[m]);
                    if (lane == 0) y_rows[(size_t)outr[m] * H + row] = v * rs;
                }
            }
        }
    }
}

// ----------------------------------------------------------------- combine
// y[t][c] = shared[t][c] + rs * sum_j w[t][j] * y_rows[t*k + j][c], slot order.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_rows,
                                                      const float* __restrict__ w, int T, int k,
                                                      int H, int has_shared, float rs,
                                                      float* __restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)T * H) return;
    const int t = (int)(i / H), c = (int)(i % H);
    float acc = 0.f;
    for (int j = 0; j < k; ++j)
        acc = fmaf(w[(int64_t)t * k + j], y_rows[((int64_t)t * k + j) * H + c], acc);
    const float sh = has_shared ? y_rows[((int64_t)T * k + t) * H + c] : 0.f;
    y[i] = fmaf(rs, acc, sh);
}

template <int W, int NCH, int MT, bool GS>
void launch_gateup_t(dim3 grid, hipStream_t s, const WorkItem* items, const int32_t* n_items,
                     const int32_t* rows_tok, const int32_t* rows_out, const uint32_t* xp,
                     const float* xs, uint32_t* hp, float* hs, int H, int I, BlobLayout L) {
    hipLaunchKernelGGL((gateup_kernel<W, NCH, MT, GS>), grid, dim3(64 * W), 0, s, items, n_items,
                       rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
}

template <int W, int NCH, bool GS>
void gateup_mt(int mt, dim3 grid, hipStream_t s, const WorkItem* items, const int32_t* n_items,
               const int32_t* rows_tok, const int32_t* rows_out, const uint32_t* xp,
               const float* xs, uint32_t* hp, float* hs, int H, int I, BlobLayout L) {
    switch (mt) {
        case 1: launch_gateup_t<W, NCH, 1, GS>(grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L); break;
        case 2: launch_gateup_t<W, NCH, 2, GS>(grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L); break;
        case 4: launch_gateup_t<W, NCH, 4, GS>(grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L); break;
        default: launch_gateup_t<W, NCH, 8, GS>(grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L); break;
    }
}

template <bool GS>
bool gateup_dispatch(int C, int mt, dim3 grid, hipStream_t s, const WorkItem* items,
                     const int32_t* n_items, const int32_t* rows_tok, const int32_t* rows_out,
                     const uint32_t* xp, const float* xs, uint32_t* hp, float* hs, int H, int I,
                     BlobLayout L) {
    if (C <= 64) gateup_mt<1, 1, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
    else if (C <= 128) gateup_mt<2, 1, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
    else if (C <= 192) gateup_mt<3, 1, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
    else if (C <= 256) gateup_mt<4, 1, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
    else if (C <= 512) gateup_mt<4, 2, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
    else if (C <= 768) gateup_mt<4, 3, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
    else if (C <= 1024) gateup_mt<4, 4, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
    else return false;
    return true;
}

template <int NCH, int MT, bool GS>
void launch_down_t(dim3 grid, hipStream_t s, const WorkItem* items, const int32_t* n_items,
                   const int32_t* rows_out, const uint32_t* hp, const float* hs, float* y, int H,
                   int I, BlobLayout L) {
    hipLaunchKernelGGL((down_kernel<NCH, MT, GS>), grid, dim3(256), 0, s, items, n_items, rows_out,
                       hp, hs, y, H, I, L);
}

template <int NCH, bool GS>
void down_mt(int mt, dim3 grid, hipStream_t s, const WorkItem* items, const int32_t* n_items,
             const int32_t* rows_out, const uint32_t* hp, const float* hs, float* y, int H, int I,
             BlobLayout L) {
    switch (mt) {
        case 1: launch_down_t<NCH, 1, GS>(grid, s, items, n_items, rows_out, hp, hs, y, H, I, L); break;
        case 2: launch_down_t<NCH, 2, GS>(grid, s, items, n_items, rows_out, hp, hs, y, H, I, L); break;
        case 4: launch_down_t<NCH, 4, GS>(grid, s, items, n_items, rows_out, hp, hs, y, H, I, L); break;
        default: launch_down_t<NCH, 8, GS>(grid, s, items, n_items, rows_out, hp, hs, y, H, I, L); break;
    }
}

template <bool GS>
bool down_dispatch(int CI, int mt, dim3 grid, hipStream_t s, const WorkItem* items,
                   const int32_t* n_items, const int32_t* rows_out, const uint32_t* hp,
                   const float* hs, float* y, int H, int I, BlobLayout L) {
    const int nch = (CI + 63) / 64;
    switch (nch) {
        case 1: down_mt<1, GS>(mt, grid, s, items, n_items, rows_out, hp, hs, y, H, I, L); break;
        case 2: down_mt<2, GS>(mt, grid, s, items, n_items, rows_out, hp, hs, y, H, I, L); break;
        case 3: down_mt<3, GS>(mt, grid, s, items, n_items, rows_out, hp, hs, y, H, I, L); break;
        case 4: down_mt<4, GS>(mt, grid, s, items, n_items, rows_out, hp, hs, y, H, I, L); break;
        default: return false;
    }
    return true;
}

}  // namespace

coli_status launch_encode(const float* x, int32_t rows, int32_t K, uint32_t* planes, float* scales,
                          hipStream_t stream) {
    if (rows == 0) return COLI_OK;
    const int64_t threads = (int64_t)rows * (K / kBlock) * 4;
    hipLaunchKernelGGL(encode_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                       x, rows, K, planes, scales);
    COLI_CHECK_LAUNCH("encode kernel launch");
    return COLI_OK;
}

coli_status launch_gemv_ffn(const WorkItem* items, const int32_t* n_items, int32_t max_items,
                            int32_t max_count, const int32_t* rows_tok, const int32_t* rows_out,
                            const uint32_t* xplanes, const float* xscale, uint32_t* hplanes,
                            float* hscale, float* y_rows, int32_t H, int32_t I, int32_t group,
                            hipStream_t stream) {
    if (max_items == 0) return COLI_OK;
    const BlobLayout L = blob_layout(H, I, group);
    const int mt = max_count <= 1 ? 1 : max_count <= 2 ? 2 : max_count <= 4 ? 4 : 8;
    const int C = H / kBlock, CI = I / kBlock;
    const dim3 g1(I / kBlock, max_items);
    bool ok;
    {
    ProfScope prof("gemv_gateup", stream);
    ok = group ? gateup_dispatch<true>(C, mt, g1, stream, items, n_items, rows_tok, rows_out,
                                            xplanes, xscale, hplanes, hscale, H, I, L)
                    : gateup_dispatch<false>(C, mt, g1, stream, items, n_items, rows_tok, rows_out,
                                             xplanes, xscale, hplanes, hscale, H, I, L);
    }
    if (!ok) return fail(COLI_EUNSUPPORTED, "gemv: hidden too large (max 32768)");
    COLI_CHECK_LAUNCH("gate/up GEMV launch");
    const dim3 g2((H + kDownRowsPerBlock - 1) / kDownRowsPerBlock, max_items);
    {
    ProfScope prof("gemv_down", stream);
    ok = group ? down_dispatch<true>(CI, mt, g2, stream, items, n_items, rows_out, hplanes, hscale,
                                     y_rows, H, I, L)
               : down_dispatch<false>(CI, mt, g2, stream, items, n_items, rows_out, hplanes, hscale,
                                      y_rows, H, I, L);
    }
    if (!ok) return fail(COLI_EUNSUPPORTED, "gemv: inter too large (max 8192)");
    COLI_CHECK_LAUNCH("down GEMV launch");
    return COLI_OK;
}

coli_status launch_combine(const float* y_rows, const float* w, int32_t T, int32_t k, int32_t H,
                           int32_t has_shared, float routed_scale, float* y, hipStream_t stream) {
    const int64_t n = (int64_t)T * H;
    if (n == 0) return COLI_OK;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       y_rows, w, T, k, H, has_shared, routed_scale, y);
    COLI_CHECK_LAUNCH("combine kernel launch");
    return COLI_OK;
}

}  // namespace coli
