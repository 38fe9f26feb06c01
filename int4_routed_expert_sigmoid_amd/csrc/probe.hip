// Read-ceiling probe: kernels that only stream bytes from HBM in the access
// patterns of the decode GEMVs (or in plain contiguous chunks) and fold them
// into one word per wave, so that a launch's duration is the practical read
// ceiling of that pattern on the device. No arithmetic of the layer; it
// backs the bandwidth ceilings the GEMV rooflines are compared with.
#include "common.h"

namespace coli {
namespace {

// XOR of a wave's words; lane 0 stores it.
__device__ __forceinline__ void fold_store(uint32_t v, uint32_t* sink) {
    v ^= (uint32_t)lane_xchg<1>((int)v);
    v ^= (uint32_t)lane_xchg<2>((int)v);
    v ^= (uint32_t)lane_xchg<4>((int)v);
    v ^= (uint32_t)lane_xchg<8>((int)v);
    v ^= (uint32_t)lane_xchg<16>((int)v);
    v ^= (uint32_t)lane_xchg<32>((int)v);
    if ((threadIdx.x & 63) == 0) sink[(size_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = v;
}

// Rows of `row_bytes` (a multiple of 16): the workgroup takes `rows_per_wg`
// consecutive rows. TPR = row_bytes / 16 threads read one row (one 16-byte
// load each); the workgroup's threads cover blockDim / TPR rows at a time, NF
// such steps per round with every load of a round issued before any is used
// (the host makes rows_per_wg a multiple of NF steps).
template <int NF>
__global__ __launch_bounds__(256) void probe_rows_kernel(const uint8_t* __restrict__ src,
                                                         int64_t n_rows, int row_bytes,
                                                         int rows_per_wg, uint32_t* __restrict__ sink) {
    const int tpr = row_bytes / 16;
    const int per_step = (int)blockDim.x / tpr;              // rows read at once by the workgroup
    const int rsub = (int)threadIdx.x / tpr, col = (int)threadIdx.x % tpr;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
    uint32_t acc = 0;
    for (int s0 = 0; s0 < rows_per_wg; s0 += per_step * NF) {
        uint4 v[NF];
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            const int64_t r = min(r0 + s0 + (int64_t)i * per_step + rsub, n_rows - 1);
            v[i] = ldg128(src + r * row_bytes + (size_t)col * 16);
        }
#pragma unroll
        for (int i = 0; i < NF; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
    fold_store(acc, sink);
}

// Contiguous chunks of `chunk` bytes per workgroup: NF loads of 16 bytes per
// thread in flight per round (the host makes chunk a multiple of NF * 4096).
template <int NF>
__global__ __launch_bounds__(256) void probe_chunks_kernel(const uint8_t* __restrict__ src,
                                                           int64_t bytes, int64_t chunk,
                                                           uint32_t* __restrict__ sink) {
    const int64_t base = (int64_t)blockIdx.x * chunk;
    const int64_t step = (int64_t)blockDim.x * 16;
    uint32_t acc = 0;
    for (int64_t o0 = 0; o0 < chunk; o0 += step * NF) {
        uint4 v[NF];
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            const int64_t o = min(base + o0 + i * step + (int64_t)threadIdx.x * 16, bytes - 16);
            v[i] = ldg128(src + o);
        }
#pragma unroll
        for (int i = 0; i < NF; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
    fold_store(acc, sink);
}

// The largest of 16, 8, 4, 2, 1 that divides n (loads in flight per round).
int pick_nf(int64_t n) {
    for (int nf = 16; nf > 1; nf >>= 1)
        if (n % nf == 0) return nf;
    return 1;
}

}  // namespace
}  // namespace coli

using namespace coli;

extern "C" {

COLI_API coli_status coli_read_probe(const void* d_src, size_t bytes, int32_t pattern,
                                     int32_t row_bytes, int32_t rows_per_wg, void* d_sink,
                                     size_t sink_bytes, void* stream) {
    if (!d_src || !d_sink || bytes < 16 || bytes % 16) return fail(COLI_EINVAL, "read_probe: bad buffer");
    if (pattern == 0) {
        // contiguous chunks: row_bytes is the chunk size
        const int64_t chunk = row_bytes;
        if (chunk <= 0 || chunk % (256 * 16)) return fail(COLI_EINVAL, "read_probe: chunk must be a multiple of 4096");
        const int64_t n_wg = ((int64_t)bytes + chunk - 1) / chunk;
        if ((size_t)n_wg * 4 * sizeof(uint32_t) > sink_bytes) return fail(COLI_EINVAL, "read_probe: sink too small");
        const int nf = pick_nf(chunk / 4096);
        const dim3 g((unsigned)n_wg), blk(256);
        const uint8_t* src = (const uint8_t*)d_src;
        uint32_t* sink = (uint32_t*)d_sink;
        hipStream_t st = (hipStream_t)stream;
        if (nf == 16) launch(probe_chunks_kernel<16>, g, blk, 0, st, src, (int64_t)bytes, chunk, sink);
        else if (nf == 8) launch(probe_chunks_kernel<8>, g, blk, 0, st, src, (int64_t)bytes, chunk, sink);
        else if (nf == 4) launch(probe_chunks_kernel<4>, g, blk, 0, st, src, (int64_t)bytes, chunk, sink);
        else if (nf == 2) launch(probe_chunks_kernel<2>, g, blk, 0, st, src, (int64_t)bytes, chunk, sink);
        else launch(probe_chunks_kernel<1>, g, blk, 0, st, src, (int64_t)bytes, chunk, sink);
    } else if (pattern == 1) {
        if (row_bytes <= 0 || row_bytes % 16 || (row_bytes / 16 > 256) || (256 % (row_bytes / 16) && row_bytes / 16 != 192))
            return fail(COLI_EINVAL, "read_probe: row_bytes / 16 must divide 256 or be 192");
        if (rows_per_wg <= 0 || bytes % (size_t)row_bytes) return fail(COLI_EINVAL, "read_probe: bad rows");
        const int tpr = row_bytes / 16, threads = tpr == 192 ? 192 : 256;
        const int64_t n_rows = (int64_t)(bytes / (size_t)row_bytes);
        const int64_t n_wg = (n_rows + rows_per_wg - 1) / rows_per_wg;
        if ((size_t)n_wg * (threads / 64) * sizeof(uint32_t) > sink_bytes) return fail(COLI_EINVAL, "read_probe: sink too small");
        const int per_step = threads / tpr;
        if (rows_per_wg % per_step) return fail(COLI_EINVAL, "read_probe: rows_per_wg must be a multiple of the rows read at once");
        const int nf = pick_nf(rows_per_wg / per_step);
        const dim3 g((unsigned)n_wg), blk((unsigned)threads);
        const uint8_t* src = (const uint8_t*)d_src;
        uint32_t* sink = (uint32_t*)d_sink;
        hipStream_t st = (hipStream_t)stream;
        if (nf == 16) launch(probe_rows_kernel<16>, g, blk, 0, st, src, n_rows, row_bytes, rows_per_wg, sink);
        else if (nf == 8) launch(probe_rows_kernel<8>, g, blk, 0, st, src, n_rows, row_bytes, rows_per_wg, sink);
        else if (nf == 4) launch(probe_rows_kernel<4>, g, blk, 0, st, src, n_rows, row_bytes, rows_per_wg, sink);
        else if (nf == 2) launch(probe_rows_kernel<2>, g, blk, 0, st, src, n_rows, row_bytes, rows_per_wg, sink);
        else launch(probe_rows_kernel<1>, g, blk, 0, st, src, n_rows, row_bytes, rows_per_wg, sink);
    } else {
        return fail(COLI_EINVAL, "read_probe: pattern must be 0 (chunks) or 1 (rows)");
    }
    COLI_CHECK_LAUNCH("read probe launch");
    return COLI_OK;
}

}  // extern "C"
