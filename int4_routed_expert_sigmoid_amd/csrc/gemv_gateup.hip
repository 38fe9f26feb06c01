// gate/up half of the int4 GEMV family (decode and small per-expert counts).
//
// Expert FFN (practical guide section 二: gate, up and down stored adjacently;
// SwiGLU): h = silu(gate x) * (up x) for every (expert, token) pair of a work
// list, each expert's gate and up rows streamed once per pass of up to MT
// tokens.
//
// Workgroup: 32 rows (one h block) of one work item's gate and up matrices.
// W waves split the reduction axis: thread tid owns the 32-column blocks
// tid + 64*W*j and reads the 16 bytes of each row that fall in them with
// one 128-bit load. Each block's nibbles are multiplied by the token's digit
// planes with v_dot8_i32_i4 (exact int32 per block, common.h) and scaled
// once into an f32 partial. Rows go in batches of LB = 4/MT rows: a batch
// yields 2*LB*MT partials per lane, summed over the wave by one
// transpose-reduction and over the W waves through LDS; the next batch's
// loads are issued before the current batch is computed. The workgroup ends
// by applying SiLU, multiplying, and encoding the 32 h values of each token
// as one digit block for the down pass.
#include "gemv.h"

namespace coli {
namespace {

// Resident waves per SIMD the register budget must allow: the decode grid
// (9 work items x 64 tiles) then fits on the chip in one round.
template <int NCH, int MT, bool GS>
constexpr int gateup_waves_per_eu() {
    return NCH == 1 && MT <= 4 && (!GS || MT >= 2) ? 3 : 2;
}

template <int W, int NCH, int MT, bool GS>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(gateup_waves_per_eu<NCH, MT, GS>(), 8)))
void gateup_kernel(
    const WorkItem* __restrict__ items, const int32_t* __restrict__ n_items,
    const int32_t* __restrict__ rows_tok, const int32_t* __restrict__ rows_out,
    const uint32_t* __restrict__ xplanes, const float* __restrict__ xscale,
    uint32_t* __restrict__ hplanes, float* __restrict__ hscale, int H, int I, BlobLayout L) {
    constexpr int LB = (4 / MT) > 0 ? (4 / MT) : 1;   // rows per batch
    constexpr int NV = 2 * LB * MT;                   // partials per batch (8, or 16 for MT 8)
    constexpr int SH = transpose_shift<NV>();
    constexpr int NBT = kBlock / LB;                  // batches per tile (even)
    static_assert(NBT % 2 == 0, "batch count must be even");
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

    __shared__ float red[W][kBlock * 2 * MT];
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

        uint4 wa[LB][2][NCH], wb[LB][2][NCH];
        float fa[LB][2][NCH], fb[LB][2][NCH];
        auto load = [&](uint4 (&wv)[LB][2][NCH], float (&fv)[LB][2][NCH], int batch) {
#pragma unroll
            for (int r = 0; r < LB; ++r) {
                const int row = r0 + batch * LB + r;
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    // unconditional loads (no branch for the wait-count pass to
                    // merge at): threads past the row end re-read its last block,
                    // and their digit planes and scales are zero
                    const int ch = min(tid + 64 * W * j, C - 1);
                    wv[r][0][j] = ldg128(gq + row * rowbytes + (size_t)ch * 16);
                    wv[r][1][j] = ldg128(uq + row * rowbytes + (size_t)ch * 16);
                    if (GS) {
                        fv[r][0][j] = ldg_f32(gsc + (size_t)row * gpr + (ch >> 1));
                        fv[r][1][j] = ldg_f32(usc + (size_t)row * gpr + (ch >> 1));
                    }
                }
            }
        };
        auto compute = [&](const uint4 (&wv)[LB][2][NCH], const float (&fv)[LB][2][NCH], int batch) {
            float part[NV];
#pragma unroll
            for (int r = 0; r < LB; ++r)
#pragma unroll
                for (int mat = 0; mat < 2; ++mat)
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        float acc = 0.f;
                        if (m < mc) {
#pragma unroll
                            for (int j = 0; j < NCH; ++j) {
                                const float f = GS ? xs[m][j] * fv[r][mat][j] : xs[m][j];
                                acc += (float)block_dot(wv[r][mat][j], xp[m][j]) * f;
                            }
                        }
                        part[(r * 2 + mat) * MT + m] = acc;
                    }
            const float v = wave_transpose_sum<NV>(part);
            if ((lane & ((1 << SH) - 1)) == 0)
                red[wave][batch * NV + (lane >> SH)] = v;
        };
        load(wa, fa, 0);
#pragma unroll 1
        for (int b = 0; b < NBT; b += 2) {
            load(wb, fb, b + 1);
            compute(wa, fa, b);
            if (b + 2 < NBT) load(wa, fa, b + 2);
            compute(wb, fb, b + 1);
        }
        __syncthreads();
        for (int i = tid; i < kBlock * MT; i += 64 * W) {
            const int r = i / MT, m = i % MT;
            if (m < mc) {
                float g = 0.f, u = 0.f;
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    g += red[w][(r * 2 + 0) * MT + m];
                    u += red[w][(r * 2 + 1) * MT + m];
                }
                if (!GS) { g *= ldg_f32(gsc + r0 + r); u *= ldg_f32(usc + r0 + r); }
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

template <int W, int NCH, int MT, bool GS>
void launch_t(dim3 grid, hipStream_t s, const WorkItem* items, const int32_t* n_items,
              const int32_t* rows_tok, const int32_t* rows_out, const uint32_t* xp,
              const float* xs, uint32_t* hp, float* hs, int H, int I, const BlobLayout& L) {
    launch((gateup_kernel<W, NCH, MT, GS>), grid, dim3(64 * W), 0, s, items, n_items,
                       rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
}

template <int W, int NCH, bool GS>
void by_mt(int mt, dim3 grid, hipStream_t s, const WorkItem* items, const int32_t* n_items,
           const int32_t* rows_tok, const int32_t* rows_out, const uint32_t* xp, const float* xs,
           uint32_t* hp, float* hs, int H, int I, const BlobLayout& L) {
    switch (mt) {
        case 1: launch_t<W, NCH, 1, GS>(grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L); break;
        case 2: launch_t<W, NCH, 2, GS>(grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L); break;
        case 4: launch_t<W, NCH, 4, GS>(grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L); break;
        default: launch_t<W, NCH, 8, GS>(grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L); break;
    }
}

template <bool GS>
bool by_width(int C, int mt, dim3 grid, hipStream_t s, const WorkItem* items,
              const int32_t* n_items, const int32_t* rows_tok, const int32_t* rows_out,
              const uint32_t* xp, const float* xs, uint32_t* hp, float* hs, int H, int I,
              const BlobLayout& L) {
    if (C <= 64) by_mt<1, 1, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
    else if (C <= 128) by_mt<2, 1, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
    else if (C <= 192) by_mt<3, 1, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
    else if (C <= 256) by_mt<4, 1, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
    else if (C <= 512) by_mt<4, 2, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L);
    else return false;
    return true;
}

}  // namespace

bool dispatch_gateup(int mt, int group, dim3 grid, hipStream_t s, const WorkItem* items,
                     const int32_t* n_items, const int32_t* rows_tok, const int32_t* rows_out,
                     const uint32_t* xplanes, const float* xscale, uint32_t* hplanes,
                     float* hscale, int H, int I, const BlobLayout& L) {
    const int C = H / kBlock;
    return group ? by_width<true>(C, mt, grid, s, items, n_items, rows_tok, rows_out, xplanes,
                                  xscale, hplanes, hscale, H, I, L)
                 : by_width<false>(C, mt, grid, s, items, n_items, rows_tok, rows_out, xplanes,
                                   xscale, hplanes, hscale, H, I, L);
}

}  // namespace coli
