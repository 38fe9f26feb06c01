// down half of the int4 GEMV family: y_e = down_e h for every (expert, token)
// pair of a work list (practical guide section 二: gate, up, down adjacent).
//
// Workgroup: 4 waves x 16 rows of one work item's down matrix. Lane l owns
// the 32-column blocks l + 64*j of h (the digit blocks written by the gate/up
// pass) and reads each row's 16 bytes in those blocks with one 128-bit load.
// Rows go in batches of LB = 4/MT rows whose LB*MT partials per lane are
// summed over the wave by one transpose-reduction; the next batch's loads are
// issued before the current batch is computed.
#include "gemv.h"

namespace coli {
namespace {

template <int NCH, int MT, bool GS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NCH == 1 && MT <= 4 ? 4 : 2, 8)))
void down_kernel(
    const WorkItem* __restrict__ items, const int32_t* __restrict__ n_items,
    const int32_t* __restrict__ rows_out, const uint32_t* __restrict__ hplanes,
    const float* __restrict__ hscale, float* __restrict__ y_rows, int H, int I, BlobLayout L) {
    constexpr int LB = (4 / MT) > 0 ? (4 / MT) : 1;      // rows per batch
    constexpr int NV = LB * MT;                          // partials per batch (4, or 8 for MT 8)
    constexpr int SH = transpose_shift<NV>();
    constexpr int NBT = kDownRowsPerWave / LB;           // batches per wave (even)
    static_assert(NBT % 2 == 0, "batch count must be even");
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

    for (int m0 = 0; m0 < it.count && rbase < H; m0 += MT) {
        const int mc = min(MT, it.count - m0);
        uint4 hp[MT][NCH][kPlanes];
        float hs[MT][NCH];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int outr = (m < mc) ? rows_out[it.begin + m0 + m] : 0;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int ch = lane + 64 * j;
                if (m < mc && ch < CI) {
                    const uint4* src = reinterpret_cast<const uint4*>(
                        hplanes + ((size_t)outr * CI + ch) * kWordsPerBlock);
#pragma unroll
                    for (int p = 0; p < kPlanes; ++p) hp[m][j][p] = src[p];
                    hs[m][j] = hscale[(size_t)outr * CI + ch];
                } else {
#pragma unroll
                    for (int p = 0; p < kPlanes; ++p) hp[m][j][p] = make_uint4(0, 0, 0, 0);
                    hs[m][j] = 0.f;
                }
            }
        }
        uint4 wa[LB][NCH], wb[LB][NCH];
        float fa[LB][NCH], fb[LB][NCH];
        auto load = [&](uint4 (&wv)[LB][NCH], float (&fv)[LB][NCH], int batch) {
#pragma unroll
            for (int r = 0; r < LB; ++r) {
                const int row = min(rbase + batch * LB + r, H - 1);   // rows past H: dropped
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    // unconditional loads: lanes past the row end re-read its last
                    // block; their digit planes and scales are zero
                    const int ch = min(lane + 64 * j, CI - 1);
                    wv[r][j] = ldg128(dq + row * rowbytes + (size_t)ch * 16);
                    if (GS) fv[r][j] = ldg_f32(dsc + (size_t)row * gpr + (ch >> 1));
                }
            }
        };
        auto compute = [&](const uint4 (&wv)[LB][NCH], const float (&fv)[LB][NCH], int batch) {
            float part[NV];
#pragma unroll
            for (int r = 0; r < LB; ++r)
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    float acc = 0.f;
                    if (m < mc) {
#pragma unroll
                        for (int j = 0; j < NCH; ++j) {
                            const float f = GS ? hs[m][j] * fv[r][j] : hs[m][j];
                            acc += (float)block_dot(wv[r][j], hp[m][j]) * f;
                        }
                    }
                    part[r * MT + m] = acc;
                }
            const float v = wave_transpose_sum<NV>(part);
            const int vi = lane >> SH;
            const int r = vi / MT, m = vi % MT;
            const int row = rbase + batch * LB + r;
            if ((lane & ((1 << SH) - 1)) == 0 && m < mc && row < H) {
                const int outr = rows_out[it.begin + m0 + m];
                y_rows[(size_t)outr * H + row] = v * (GS ? 1.f : ldg_f32(dsc + row));
            }
        };
        load(wa, fa, 0);
#pragma unroll 1
        for (int b = 0; b < NBT; b += 2) {
            load(wb, fb, b + 1);
            compute(wa, fa, b);
            if (b + 2 < NBT) load(wa, fa, b + 2);
            compute(wb, fb, b + 1);
        }
    }
}

template <int NCH, int MT, bool GS>
void launch_t(dim3 grid, hipStream_t s, const WorkItem* items, const int32_t* n_items,
              const int32_t* rows_out, const uint32_t* hp, const float* hs, float* y, int H,
              int I, const BlobLayout& L) {
    launch((down_kernel<NCH, MT, GS>), grid, dim3(256), 0, s, items, n_items, rows_out,
           hp, hs, y, H, I, L);
}

template <int NCH, bool GS>
void by_mt(int mt, dim3 grid, hipStream_t s, const WorkItem* items, const int32_t* n_items,
           const int32_t* rows_out, const uint32_t* hp, const float* hs, float* y, int H, int I,
           const BlobLayout& L) {
    switch (mt) {
        case 1: launch_t<NCH, 1, GS>(grid, s, items, n_items, rows_out, hp, hs, y, H, I, L); break;
        case 2: launch_t<NCH, 2, GS>(grid, s, items, n_items, rows_out, hp, hs, y, H, I, L); break;
        case 4: launch_t<NCH, 4, GS>(grid, s, items, n_items, rows_out, hp, hs, y, H, I, L); break;
        default: launch_t<NCH, 8, GS>(grid, s, items, n_items, rows_out, hp, hs, y, H, I, L); break;
    }
}

template <bool GS>
bool by_width(int CI, int mt, dim3 grid, hipStream_t s, const WorkItem* items,
              const int32_t* n_items, const int32_t* rows_out, const uint32_t* hp,
              const float* hs, float* y, int H, int I, const BlobLayout& L) {
    const int nch = (CI + 63) / 64;
    if (nch == 1) by_mt<1, GS>(mt, grid, s, items, n_items, rows_out, hp, hs, y, H, I, L);
    else if (nch == 2) by_mt<2, GS>(mt, grid, s, items, n_items, rows_out, hp, hs, y, H, I, L);
    else return false;
    return true;
}

}  // namespace

bool dispatch_down(int mt, int group, dim3 grid, hipStream_t s, const WorkItem* items,
                   const int32_t* n_items, const int32_t* rows_out, const uint32_t* hplanes,
                   const float* hscale, float* y_rows, int H, int I, const BlobLayout& L) {
    const int CI = I / kBlock;
    return group ? by_width<true>(CI, mt, grid, s, items, n_items, rows_out, hplanes, hscale,
                                  y_rows, H, I, L)
                 : by_width<false>(CI, mt, grid, s, items, n_items, rows_out, hplanes, hscale,
                                   y_rows, H, I, L);
}

}  // namespace coli
