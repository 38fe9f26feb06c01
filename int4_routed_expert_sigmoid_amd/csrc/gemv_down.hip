// down half of the int4 GEMV family: y_e = down_e h for every (expert, token)
// pair of a work list (practical guide section 二: gate, up, down adjacent;
// SwiGLU), with h = silu(g) * u as the gate/up pass encoded it: digit planes
// of 16-element blocks, two per 32-column block of a down row (common.h,
// kHBlock).
//
// Workgroup: 4 waves x RPW rows of one work item's down matrix (8 for one-token
// launches, 16 for batches). Lane l owns the 32-column blocks l + 64*j of h
// and reads each row's 16 bytes in those blocks with one 128-bit load. Rows
// go in batches of LB = 4/MT rows whose LB*MT partials per lane are summed
// over the wave by one transpose-reduction; loads run two batches ahead (one
// token: every row of the wave requested at once) or one batch ahead
// (batches). The h blocks and row scales are requested before the weights.
#include <algorithm>

#include "gemv.h"

namespace coli {
namespace {

// One work item's rows of this workgroup for all of its tokens, MT at a time.
// ONE (one-token launches): the item's output row is its h row.
template <int NCH, int MT, bool GS, bool ONE, bool W8>
__device__ __forceinline__ void down_body(
    const WorkItem& it, const int32_t* __restrict__ rows_out,
    const uint32_t* __restrict__ hplanes, const float* __restrict__ hscale,
    float* __restrict__ y_rows, int H, int I, const BlobLayout& L) {
    constexpr int LB = (4 / MT) > 0 ? (4 / MT) : 1;      // rows per batch
    constexpr int NV = LB * MT;                          // partials per batch (4, or 8 for MT 8)
    constexpr int SH = transpose_shift<NV>();
    constexpr int RPW = down_rows_per_wave(ONE ? 1 : 4); // rows per wave
    constexpr int NBT = RPW / LB;                        // batches per wave
    constexpr int PD = (NCH == 1 && ONE) ? 3 : 2;        // weight register sets (prefetch depth + 1)
    const int CI = I / kBlock;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rbase = (blockIdx.x * 4 + wave) * RPW;
    if (rbase >= H) return;                              // wave-uniform; no barriers below
    const uint8_t* dq = it.blob + L.down_q;
    const float* dsc = reinterpret_cast<const float*>(it.blob + L.down_s);
    const size_t rowbytes = (size_t)I / (W8 ? 1 : 2);
    const int gpr = GS ? I / 64 : 1;

    int rowwin = 0;                                      // output rows of a 64-token window, one per lane
    const int count = ONE ? 1 : it.count;                // one-token items: a constant trip count
    for (int m0 = 0; m0 < count; m0 += MT) {
        const int mc = ONE ? 1 : min(MT, count - m0);
        if (!ONE && (m0 & 63) == 0) rowwin = rows_out[it.begin + min(m0 + lane, it.count - 1)];
        // the h blocks of the chunk's tokens and the per-row scales of the
        // wave's rows (lane l: row rbase + l % RPW) first: load counters
        // retire in order, so the first batch then waits for them and its own
        // weights alone
        uint4 hp[MT][NCH][kPlanes];
        float2 hs[MT][NCH];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int outr = ONE ? it.row0 : __builtin_amdgcn_readlane(rowwin, (m0 & 63) + min(m, mc - 1));
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                // unconditional loads (clamped token and block); tokens and
                // blocks past the end are masked where the partials are formed
                const size_t blk = (size_t)outr * CI + min(lane + 64 * j, CI - 1);
                const uint4* src = reinterpret_cast<const uint4*>(hplanes + blk * kWordsPerBlock);
#pragma unroll
                for (int p = 0; p < kPlanes; ++p) hp[m][j][p] = src[p];
                hs[m][j] = *reinterpret_cast<const float2*>(hscale + blk * 2);
            }
        }
        const float rsc = GS ? 1.f : ldg_f32(dsc + min(rbase + (lane % RPW), H - 1));
        WBlock<W8> wbuf[PD][LB][NCH];
        float fbuf[PD][LB][NCH];
        auto load = [&](WBlock<W8> (&wv)[LB][NCH], float (&fv)[LB][NCH], int batch) {
#pragma unroll
            for (int r = 0; r < LB; ++r) {
                const int row = min(rbase + batch * LB + r, H - 1);   // rows past H: dropped
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    // unconditional loads: lanes past the row end re-read its last
                    // block; their products are masked
                    const int ch = min(lane + 64 * j, CI - 1);
                    wv[r][j] = load_wblock<W8>(dq + row * rowbytes, ch);
                    if (GS) fv[r][j] = ldg_f32(dsc + (size_t)row * gpr + (ch >> 1));
                }
            }
        };
#pragma unroll
        for (int b = 0; b < PD - 1; ++b) load(wbuf[b], fbuf[b], b);
        sched_fence();    // keep these loads ahead of the waits below
        int2 hsum[MT][NCH];                              // int8 weights: sums of each half's X
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int j = 0; j < NCH; ++j) hsum[m][j] = W8 ? digit_sum_halves(hp[m][j]) : make_int2(0, 0);
        auto compute = [&](const WBlock<W8> (&wv)[LB][NCH], const float (&fv)[LB][NCH], int batch) {
            float part[NV];
#pragma unroll
            for (int r = 0; r < LB; ++r)
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    float acc = 0.f;
                    if (m < mc) {
#pragma unroll
                        for (int j = 0; j < NCH; ++j) {
                            // blocks past the row end add nothing (mask on the product,
                            // so that it is not hoisted with a wait for hs)
                            const float fa = GS ? hs[m][j].x * fv[r][j] : hs[m][j].x;
                            const float fb = GS ? hs[m][j].y * fv[r][j] : hs[m][j].y;
                            const int2 d = wblock_dot_halves<W8>(wv[r][j], hp[m][j], hsum[m][j]);
                            const float t = fmaf((float)d.x, fa, (float)d.y * fb);
                            acc += lane + 64 * j < CI ? t : 0.f;
                        }
                    }
                    part[r * MT + m] = acc;
                }
            const float v = wave_transpose_sum<NV>(part);
            const int vi = lane >> SH;
            const int r = vi / MT, m = vi % MT;
            const int row = rbase + batch * LB + r;
            // scale and output row from registers (a global load here would
            // wait for the prefetched weights)
            const float sc = GS ? 1.f : __shfl(rsc, batch * LB + r);
            const int outr = ONE ? it.row0 : __shfl(rowwin, (m0 & 63) + m);
            if ((lane & ((1 << SH) - 1)) == 0 && m < mc && row < H)
                y_rows[(size_t)outr * H + row] = v * sc;
        };
        // each batch's loads are issued before the wait for an earlier one;
        // the scheduling fences keep the scheduler from moving a wait
        // above them, and no load is left under a runtime condition (the
        // wait-count pass would merge it by draining the batch in flight)
        if constexpr (PD == 3) {
#pragma unroll
            for (int b = 0; b < NBT; ++b) {
                if (b + 2 < NBT) load(wbuf[(b + 2) % 3], fbuf[(b + 2) % 3], b + 2);
                sched_fence();
                compute(wbuf[b % 3], fbuf[b % 3], b);
            }
        } else {
            static_assert(NBT % 2 == 0, "batch count must be even");
#pragma unroll 1
            for (int b = 0; b < NBT - 2; b += 2) {
                load(wbuf[1], fbuf[1], b + 1);
                sched_fence();
                compute(wbuf[0], fbuf[0], b);
                load(wbuf[0], fbuf[0], b + 2);
                sched_fence();
                compute(wbuf[1], fbuf[1], b + 1);
            }
            load(wbuf[1], fbuf[1], NBT - 1);
            sched_fence();
            compute(wbuf[0], fbuf[0], NBT - 2);
            compute(wbuf[1], fbuf[1], NBT - 1);
        }
    }
}

// MTK == 1: one token; MTK == 4: batches, each work item taking the body that
// fits its token count (1, 2, or chunks of 4).
template <int NCH, int MTK, bool GS, bool W8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(W8 ? (NCH == 1 && MTK == 1 && !GS ? 3 : 2) : NCH == 1 && MTK == 1 && !GS ? 4 : NCH == 1 ? 3 : 2, 8)))
void down_kernel(
    const WorkItem* __restrict__ items, const int32_t* __restrict__ n_items,
    const int32_t* __restrict__ rows_out, const uint32_t* __restrict__ hplanes,
    const float* __restrict__ hscale, float* __restrict__ y_rows, int H, int I, BlobLayout L,
    ReadLog rl) {
    const int item = blockIdx.y;
    if (item >= *n_items) return;
    const WorkItem it = items[item];
    if constexpr (MTK == 1) {
        down_body<NCH, 1, GS, true, W8>(it, rows_out, hplanes, hscale, y_rows, H, I, L);
        log_read(rl, it.blob, 1, blockIdx.x, 4 * down_rows_per_wave(1), 1);
    } else {
        log_read(rl, it.blob, 1, blockIdx.x, 4 * down_rows_per_wave(4),
                 it.count <= 2 ? 1 : (it.count + 3) / 4);
        if (it.count == 1) down_body<NCH, 1, GS, false, W8>(it, rows_out, hplanes, hscale, y_rows, H, I, L);
        else if (it.count == 2) down_body<NCH, 2, GS, false, W8>(it, rows_out, hplanes, hscale, y_rows, H, I, L);
        else down_body<NCH, 4, GS, false, W8>(it, rows_out, hplanes, hscale, y_rows, H, I, L);
    }
}

template <int NCH, int MT, bool GS>
void launch_t(dim3 grid, hipStream_t s, const WorkItem* items, const int32_t* n_items,
              const int32_t* rows_out, const uint32_t* hp, const float* hs, float* y, int H,
              int I, const BlobLayout& L, const ReadLog& rl) {
    if (L.wbits == 8)
        launch((down_kernel<NCH, MT, GS, true>), grid, dim3(256), 0, s, items, n_items, rows_out,
               hp, hs, y, H, I, L, rl);
    else
        launch((down_kernel<NCH, MT, GS, false>), grid, dim3(256), 0, s, items, n_items, rows_out,
               hp, hs, y, H, I, L, rl);
}

template <int NCH, bool GS>
void by_mt(int mt, dim3 grid, hipStream_t s, const WorkItem* items, const int32_t* n_items,
           const int32_t* rows_out, const uint32_t* hp, const float* hs, float* y, int H, int I,
           const BlobLayout& L, const ReadLog& rl) {
    if (mt == 1) launch_t<NCH, 1, GS>(grid, s, items, n_items, rows_out, hp, hs, y, H, I, L, rl);
    else launch_t<NCH, 4, GS>(grid, s, items, n_items, rows_out, hp, hs, y, H, I, L, rl);
}

template <bool GS>
bool by_width(int CI, int mt, dim3 grid, hipStream_t s, const WorkItem* items,
              const int32_t* n_items, const int32_t* rows_out, const uint32_t* hp,
              const float* hs, float* y, int H, int I, const BlobLayout& L,
              const ReadLog& rl) {
    const int nch = (CI + 63) / 64;
    if (nch == 1) by_mt<1, GS>(mt, grid, s, items, n_items, rows_out, hp, hs, y, H, I, L, rl);
    else if (nch == 2) by_mt<2, GS>(mt, grid, s, items, n_items, rows_out, hp, hs, y, H, I, L, rl);
    else return false;
    return true;
}

}  // namespace

bool dispatch_down(int mt, int group, dim3 grid, hipStream_t s, const WorkItem* items,
                   const int32_t* n_items, const int32_t* rows_out, const uint32_t* hplanes,
                   const float* hscale, float* y_rows, int H, int I, const BlobLayout& L,
                   const ReadLog& rl) {
    const int CI = I / kBlock;
    return group ? by_width<true>(CI, mt, grid, s, items, n_items, rows_out, hplanes, hscale,
                                  y_rows, H, I, L, rl)
                 : by_width<false>(CI, mt, grid, s, items, n_items, rows_out, hplanes, hscale,
                                   y_rows, H, I, L, rl);
}

}  // namespace coli
