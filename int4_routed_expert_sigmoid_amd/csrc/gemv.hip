// int4 dequant GEMV family for decode and small per-expert token counts:
// encoding of x, the launch of the gate/up and down passes (gemv_gateup.hip,
// gemv_down.hip) and the slot-order combine.
//
// Expert FFN (practical guide section 二: gate, up and down stored adjacently;
// SwiGLU): h = silu(gate x) * (up x), y = down h, for every (expert, token)
// pair of a work list, each expert's weights streamed once per pass of up to
// MT tokens.
#include <algorithm>

#include "gemv.h"

namespace coli {
namespace {

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

// Digit planes of the x rows a work list reads (launch_encode_items). Thread
// (m, block, quarter) of item blockIdx.y; the four quarters of a block are
// adjacent lanes and leave together when m is past the item's tokens.
__global__ __launch_bounds__(256) void encode_items_kernel(const WorkItem* __restrict__ items,
                                                           const int32_t* __restrict__ n_items,
                                                           const int32_t* __restrict__ rows_idx,
                                                           const float* __restrict__ x, int K,
                                                           uint32_t* __restrict__ planes,
                                                           float* __restrict__ scales) {
    if ((int)blockIdx.y >= *n_items) return;
    const WorkItem it = items[blockIdx.y];
    const int C = K / kBlock;
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int m = (int)(g / (C * 4)), rem = (int)(g % (C * 4));
    if (m >= it.count) return;
    const int row = rows_idx[it.begin + m];
    const int blk = rem >> 2, q = rem & 3;
    float v[8];
    const float* p = x + (size_t)row * K + blk * kBlock + q * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = p[e];
    uint32_t words[kPlanes];
    const float sc = encode_quarter(v, words);
    uint32_t* dst = planes + ((size_t)row * C + blk) * kWordsPerBlock;
#pragma unroll
    for (int p = 0; p < kPlanes; ++p) dst[p * 4 + q] = words[p];
    if (q == 0) scales[(size_t)row * C + blk] = sc;
}

// ----------------------------------------------------------------- combine
// y[t][c] = shared[t][c] + rs * sum_j w[t][j] * y_rows[t*k + j][c], slot order.
// Grid: (column blocks of 256, tokens); the slot loads are issued in groups of
// 8 before their multiply-adds, which keep the slot order.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_rows,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ idx, int T,
                                                      int k, int H, int has_shared, float rs,
                                                      float* __restrict__ y) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= H) return;
    for (int t = blockIdx.y; t < T; t += gridDim.y) {
        const float* wt = w + (int64_t)t * k;
        const int32_t* it = idx + (int64_t)t * k;
        const float* yr = y_rows + (int64_t)t * k * H + c;
        const float sh = has_shared ? y_rows[((int64_t)T * k + t) * H + c] : 0.f;
        float acc = 0.f;
        int j = 0;
        for (; j + 8 <= k; j += 8) {
            float wv[8], yv[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                wv[q] = wt[j + q];
                yv[q] = yr[(int64_t)(j + q) * H];
            }
            if (idx) {
                // a slot dropped by top-p has no output row: it adds nothing
#pragma unroll
                for (int q = 0; q < 8; ++q) yv[q] = it[j + q] < 0 ? 0.f : yv[q];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) acc = fmaf(wv[q], yv[q], acc);
        }
        for (; j < k; ++j) {
            const float yv = (idx && it[j] < 0) ? 0.f : yr[(int64_t)j * H];
            acc = fmaf(wt[j], yv, acc);
        }
        y[(int64_t)t * H + c] = fmaf(rs, acc, sh);
    }
}

}  // namespace

coli_status launch_encode(const float* x, int32_t rows, int32_t K, uint32_t* planes, float* scales,
                          hipStream_t stream) {
    if (rows == 0) return COLI_OK;
    const int64_t threads = (int64_t)rows * (K / kBlock) * 4;
    launch(encode_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                       x, rows, K, planes, scales);
    COLI_CHECK_LAUNCH("encode kernel launch");
    return COLI_OK;
}

coli_status launch_encode_items(const WorkItem* items, const int32_t* n_items, int32_t max_items,
                                int32_t max_count, const int32_t* rows_idx, const float* x,
                                int32_t K, uint32_t* planes, float* scales, hipStream_t stream) {
    if (max_items == 0 || max_count == 0) return COLI_OK;
    const int64_t threads = (int64_t)max_count * (K / kBlock) * 4;
    const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)max_items);
    launch(encode_items_kernel, grid, dim3(256), 0, stream, items, n_items, rows_idx, x, K, planes,
           scales);
    COLI_CHECK_LAUNCH("item encoding kernel launch");
    return COLI_OK;
}

coli_status launch_gemv_ffn(const WorkItem* items, const int32_t* n_items, int32_t max_items,
                            int32_t max_count, const int32_t* rows_tok, const int32_t* rows_out,
                            const uint32_t* xplanes, const float* xscale, uint32_t* hplanes,
                            float* hscale, float* y_rows, int32_t H, int32_t I, int32_t group,
                            int32_t wbits, const FusedRoute& fr, hipStream_t stream, int passes) {
    if (max_items == 0) return COLI_OK;
    const BlobLayout L = blob_layout(H, I, group, wbits);
    const int mt = max_count <= 1 ? 1 : max_count <= 2 ? 2 : max_count <= 4 ? 4 : 8;
    // one token: 16-row tiles of both matrices; batches: 32-row tiles
    const dim3 g1((mt == 1 ? 2 : 1) * (I / kBlock), max_items);
    bool ok = true;
    if (passes & kPassGateUp) {
        {
            ProfTag prof("gemv_gateup");
            ok = dispatch_gateup(mt, group, g1, stream, items, n_items, rows_tok, rows_out, xplanes,
                                 xscale, hplanes, hscale, H, I, L, fr, read_log_current());
        }
        if (!ok) return fail(COLI_EUNSUPPORTED, "gemv: hidden too large (max 16384)");
        COLI_CHECK_LAUNCH("gate/up GEMV launch");
    }
    if (!(passes & kPassDown)) return COLI_OK;
    const int down_rows = 4 * down_rows_per_wave(mt);
    const dim3 g2((H + down_rows - 1) / down_rows, max_items);
    {
        ProfTag prof("gemv_down");
        ok = dispatch_down(mt, group, g2, stream, items, n_items, rows_out, hplanes, hscale, y_rows,
                           H, I, L, read_log_current());
    }
    if (!ok) return fail(COLI_EUNSUPPORTED, "gemv: inter too large (max 4096)");
    COLI_CHECK_LAUNCH("down GEMV launch");
    return COLI_OK;
}

coli_status launch_combine(const float* y_rows, const float* w, const int32_t* idx, int32_t T,
                           int32_t k, int32_t H, int32_t has_shared, float routed_scale, float* y,
                           hipStream_t stream) {
    if ((int64_t)T * H == 0) return COLI_OK;
    const dim3 grid((unsigned)((H + 255) / 256), (unsigned)std::min(T, 65535));
    launch(combine_kernel, grid, dim3(256), 0, stream, y_rows, w, idx, T, k, H, has_shared,
           routed_scale, y);
    COLI_CHECK_LAUNCH("combine kernel launch");
    return COLI_OK;
}

// The weight-tile read log (coli_debug_read_log); off unless a caller sets it.
static ReadLog g_read_log = {nullptr, nullptr, 0};

ReadLog read_log_current() { return g_read_log; }

}  // namespace coli

using namespace coli;

extern "C" {

COLI_API coli_status coli_debug_read_log(uint32_t* d_count, void* d_records, int32_t capacity) {
    if (capacity < 0) return fail(COLI_EINVAL, "debug_read_log: capacity must be >= 0");
    if (d_count && capacity > 0 && !d_records)
        return fail(COLI_EINVAL, "debug_read_log: records buffer missing");
    g_read_log = d_count ? ReadLog{d_count, static_cast<uint4*>(d_records), capacity}
                         : ReadLog{nullptr, nullptr, 0};
    return COLI_OK;
}

}  // extern "C"
