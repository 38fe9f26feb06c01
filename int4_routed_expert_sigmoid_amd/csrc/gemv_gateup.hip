// gate/up half of the int4 GEMV family (decode and small per-expert counts).
//
// Expert FFN (practical guide section 二: gate, up and down stored adjacently;
// SwiGLU): g = gate x and u = up x for every (expert, token) pair of a work
// list, each expert's rows streamed once per pass of up to MT tokens, and
// h = silu(g) * u encoded for the down pass.
//
// Workgroup: a tile of consecutive rows of both of a work item's matrices, 16
// rows (one token: a decode token's 9 work items give 9 x 128 workgroups) or
// 32 (batches). W waves split the reduction axis: thread tid owns the 32-column
// blocks tid + 64*W*j and reads the 16 bytes of each row that fall in them
// with one 128-bit load. Each block's nibbles are multiplied by the token's
// digit planes with v_dot8_i32_i4 (exact int32 per block, common.h) and scaled
// once into an f32 partial. Rows go in batches of LB rows of both matrices: a
// batch yields LB*2*MT partials per lane, summed over the wave by one
// transpose-reduction and over the W waves through LDS; the next batch's
// loads are issued before the current batch is computed (the next two for
// one-token int4 tiles). The workgroup ends by applying the per-row scales,
// forming h = silu(g) * u for its rows and writing h as digit planes of
// 16-element blocks (kHBlock) with one scale each.
#include "gemv.h"

namespace coli {
namespace {

// One work item's tile of both matrices for all of its tokens, MT at a time.
// ONE: a one-token launch, where every row's token is 0 (the activation
// planes then load without waiting for the token index) and a tile has 16
// rows; batches take 32.
template <int W, int NCH, int MT, bool GS, bool ONE, bool W8>
__device__ __forceinline__ void gateup_body(
    const WorkItem& it, int tile, const int32_t* __restrict__ rows_tok,
    const int32_t* __restrict__ rows_out, const uint32_t* __restrict__ xplanes,
    const float* __restrict__ xscale, uint32_t* __restrict__ hplanes, float* __restrict__ hscale,
    int H, int I, const BlobLayout& L, float* red_raw) {
    constexpr int NM = 2;                             // gate and up
    constexpr int ROWS = ONE ? 16 : 32;               // rows of each matrix per tile
    constexpr int LB = ONE ? 2 : ((4 / MT) > 0 ? (4 / MT) : 1);   // rows per batch
    constexpr int NV = LB * NM * MT;                  // partials per batch (4 or 8)
    constexpr int SH = transpose_shift<NV>();
    constexpr int NBT = ROWS / LB;                    // batches per tile (even)
    static_assert(NBT % 2 == 0, "batch count must be even");
    const int r0 = tile * ROWS;
    const int C = H / kBlock;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint8_t* wq[NM];
    const float* wsc[NM];
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) {
        wq[mt] = it.blob + (mt ? L.up_q : L.gate_q);
        wsc[mt] = reinterpret_cast<const float*>(it.blob + (mt ? L.up_s : L.gate_s));
    }
    const size_t rowbytes = (size_t)H / (W8 ? 1 : 2);
    const int gpr = GS ? H / 64 : 1;

    float (*red)[ROWS * NM * MT] = reinterpret_cast<float (*)[ROWS * NM * MT]>(red_raw);

    // the per-row scales this thread applies in the epilogue (thread t:
    // token t / ROWS, row t % ROWS of both matrices), requested before the
    // weights: loaded where they are used, they would wait for every load
    // issued before them
    constexpr int NTH = MT * ROWS, NIT = (NTH + 64 * W - 1) / (64 * W);
    float rsg[NIT], rsu[NIT];
#pragma unroll
    for (int q = 0; q < NIT; ++q) {
        const int r = min(tid + q * 64 * W, NTH - 1) % ROWS;
        rsg[q] = GS ? 1.f : ldg_f32(wsc[0] + r0 + r);
        rsu[q] = GS ? 1.f : ldg_f32(wsc[1] + r0 + r);
    }

    int tokwin = 0, outwin = 0;                       // tokens and output rows of a 64-token window, one per lane
    // a one-token item runs the loop once (a constant trip count, so that the
    // first weight loads lead the activation loads)
    const int count = ONE ? 1 : it.count;
    for (int m0 = 0; m0 < count; m0 += MT) {
        const int mc = ONE ? 1 : min(MT, count - m0);
        if (!ONE && (m0 & 63) == 0) {
            tokwin = rows_tok[it.begin + min(m0 + lane, it.count - 1)];
            outwin = rows_out[it.begin + min(m0 + lane, it.count - 1)];
        }
        // two register sets of weights; the first batch is requested before
        // the activation planes
        WBlock<W8> wa[LB][NM][NCH], wb[LB][NM][NCH];
        float fa[LB][NM][NCH], fb[LB][NM][NCH];
        auto load = [&](WBlock<W8> (&wv)[LB][NM][NCH], float (&fv)[LB][NM][NCH], int batch) {
#pragma unroll
            for (int r = 0; r < LB; ++r) {
                const int row = r0 + batch * LB + r;
#pragma unroll
                for (int mt = 0; mt < NM; ++mt)
#pragma unroll
                    for (int j = 0; j < NCH; ++j) {
                        // unconditional loads (no branch for the wait-count pass to
                        // merge at): threads past the row end re-read its last
                        // block, and their products are masked
                        const int ch = min(tid + 64 * W * j, C - 1);
                        wv[r][mt][j] = load_wblock<W8>(wq[mt] + gu_row(row) * rowbytes, ch);
                        if (GS) fv[r][mt][j] = ldg_f32(wsc[mt] + (size_t)row * gpr + (ch >> 1));
                    }
            }
        };
        load(wa, fa, 0);
        uint4 xp[MT][NCH][kPlanes];
        float xs[MT][NCH];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            // unconditional loads (clamped token and block); tokens and blocks
            // past the end are masked where the partials are formed
            const int tok = ONE ? 0 : __builtin_amdgcn_readlane(tokwin, (m0 & 63) + min(m, mc - 1));
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int ch = tid + 64 * W * j, chc = min(ch, C - 1);
                const uint4* src = reinterpret_cast<const uint4*>(
                    xplanes + ((size_t)tok * C + chc) * kWordsPerBlock);
#pragma unroll
                for (int p = 0; p < kPlanes; ++p) xp[m][j][p] = src[p];
                xs[m][j] = xscale[(size_t)tok * C + chc];   // validity applied where it is used
            }
        }
        // the second batch is requested before anything waits for the first
        // (load counters retire in order); the scheduling fences keep the
        // scheduler from moving a wait above the next batch's loads
        load(wb, fb, 1);
        sched_fence();
        // one token, int4: a third register set keeps three batches in flight
        // (the batch count is a constant, so the sets rotate with static
        // indices; with int8 weights the third set measured slower)
        constexpr bool R3 = ONE && !W8;
        WBlock<W8> wc[LB][NM][NCH];
        float fc[LB][NM][NCH];
        if constexpr (R3) {
            load(wc, fc, 2);
            sched_fence();
        }
        int xsum[MT][NCH];                                // int8 weights: sum of each block's X
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int j = 0; j < NCH; ++j) xsum[m][j] = W8 ? digit_sum(xp[m][j]) : 0;

        auto compute = [&](const WBlock<W8> (&wv)[LB][NM][NCH], const float (&fv)[LB][NM][NCH], int batch) {
            float part[NV];
#pragma unroll
            for (int r = 0; r < LB; ++r)
#pragma unroll
                for (int mt = 0; mt < NM; ++mt)
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        float acc = 0.f;
                        if (m < mc) {
#pragma unroll
                            for (int j = 0; j < NCH; ++j) {
                                // blocks past the row end add nothing; the mask sits on the
                                // product, so it is not hoisted (with a wait for xs) above
                                // the first weight loads
                                const float f = GS ? xs[m][j] * fv[r][mt][j] : xs[m][j];
                                const float t = (float)wblock_dot<W8>(wv[r][mt][j], xp[m][j], xsum[m][j]) * f;
                                acc += tid + 64 * W * j < C ? t : 0.f;
                            }
                        }
                        part[(r * NM + mt) * MT + m] = acc;
                    }
            const float v = wave_transpose_sum<NV>(part);
            if ((lane & ((1 << SH) - 1)) == 0)
                red[wave][batch * NV + (lane >> SH)] = v;
        };
        if constexpr (R3) {
            static_assert(NBT == 8, "one-token tiles are 8 batches of 2 rows of both matrices");
            compute(wa, fa, 0); load(wa, fa, 3); sched_fence();
            compute(wb, fb, 1); load(wb, fb, 4); sched_fence();
            compute(wc, fc, 2); load(wc, fc, 5); sched_fence();
            compute(wa, fa, 3); load(wa, fa, 6); sched_fence();
            compute(wb, fb, 4); load(wb, fb, 7); sched_fence();
            compute(wc, fc, 5);
            compute(wa, fa, 6);
            compute(wb, fb, 7);
        } else {
            // the last pair peeled: no load under a condition, which the
            // wait-count pass would merge by draining the batch in flight
#pragma unroll 1
            for (int b = 0; b < NBT - 2; b += 2) {
                compute(wa, fa, b);
                load(wa, fa, b + 2);
                sched_fence();
                compute(wb, fb, b + 1);
                load(wb, fb, b + 3);
                sched_fence();
            }
            compute(wa, fa, NBT - 2);
            compute(wb, fb, NBT - 1);
        }
        __syncthreads();
        // output rows of this chunk's tokens (one-token items carry theirs:
        // rows_out may still be in flight when the routing is folded in)
        int outs[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
            outs[m] = ONE ? it.row0 : __builtin_amdgcn_readlane(outwin, (m0 & 63) + m);
        // thread t: row r = t % ROWS of token t / ROWS; the waves' partials of
        // its gate and up rows summed, the row scales applied, h = silu(g) * u
        // formed and each 16-row block encoded across its 16 lanes
        const int CI = I / kBlock;
#pragma unroll
        for (int q = 0; q < NIT; ++q) {
            const int t = tid + q * 64 * W, tc = min(t, NTH - 1);
            const int m = tc / ROWS, r = tc % ROWS;
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                g += red[w][(r * NM + 0) * MT + m];
                u += red[w][(r * NM + 1) * MT + m];
            }
            g *= rsg[q];
            u *= rsu[q];
            g = g * __builtin_amdgcn_rcpf(1.f + __expf(-g));            // silu(g)
            const float hv[1] = {g * u};
            uint32_t words[kPlanes];
            const float sc = encode_h16_lanes<kHBlock, 1, 1>(hv, r % kHBlock, words);
            if (t < NTH && (r % 8) == 0 && m < mc) {
                int out = outs[0];
#pragma unroll
                for (int mm = 1; mm < MT; ++mm) out = m == mm ? outs[mm] : out;
                const int rg = r0 + r / kHBlock * kHBlock, h16 = (rg / kHBlock) & 1;
                const size_t blk = (size_t)out * CI + rg / kBlock;
                uint32_t* dst = hplanes + blk * kWordsPerBlock;
#pragma unroll
                for (int p = 0; p < kPlanes; ++p) dst[p * 4 + h16 * 2 + ((r % kHBlock) >> 3)] = words[p];
                if (r % kHBlock == 0) hscale[blk * 2 + h16] = sc;
            }
        }
        if constexpr (!ONE) __syncthreads();   // red is reused by the next chunk
    }
}


// Work item `item` of a one-token call from the folded routing (FusedRoute).
// The shared expert's workgroups need no routing and start on their weights
// at once. In every other workgroup the first wave selects the top-k from the
// selection codes (select_topk), ranks the kept picks by expert id (the work
// list order: shared expert first, then the kept experts by id) and takes the
// workgroup's own pick, which it hands to the other waves through LDS (they
// wait at one barrier instead of repeating the selection: all workgroups of a
// decode launch are resident at once, so a selection per wave would queue
// about three of them on every SIMD before the first weight load).
// Workgroup (0, first routed item) publishes the routing, the slot-list rows
// and the item count, and each (0, item) workgroup its item, for the passes
// that follow. False: no such item (a slot dropped by top-p).
struct FusedPick {
    const uint8_t* blob;
    int begin, row0, ok;
};

__device__ __forceinline__ bool fused_item(const FusedRoute& fr, int item, WorkItem& it,
                                           FusedPick* pick) {
    constexpr int EPL = kFusedMaxExperts / 64;
    const int lane = threadIdx.x & 63;
    const int k = fr.k, base = fr.shared ? 1 : 0;
    if (item < base) {
        it.blob = (const uint8_t*)fr.shared;
        it.begin = k;
        it.count = 1;
        it.row0 = k;
        if (blockIdx.x == 0 && threadIdx.x == 0) fr.items[item] = it;
        return true;
    }
    if (threadIdx.x < 64) {
        uint64_t code[EPL];
        float score[EPL];
        const void* ptr[EPL];                        // blob pointers, loaded with the codes
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = min(lane + 64 * i, fr.E - 1);
            code[i] = fr.codes[e];
            score[i] = fr.scores[e];
            ptr[i] = fr.table[e];
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) code[i] = lane + 64 * i < fr.E ? code[i] : 0;
        const TopK r = select_topk<EPL>(code, score, k, fr.topp);
        const int kept = r.kept;
        const bool mine = lane < kept;
        int below = 0;                               // rank of this lane's pick by expert id
        for (int j = 0; j < kept; ++j) below += __builtin_amdgcn_readlane(r.my_idx, j) < r.my_idx;
        if (blockIdx.x == 0 && item == base) {
            if (lane < k) {
                fr.idx[lane] = mine ? r.my_idx : -1;
                fr.w[lane] = mine ? r.my_w : 0.f;
            }
            if (mine) {
                fr.rows_tok[below] = 0;
                fr.rows_out[below] = lane;
            }
            if (lane == 0) {
                fr.rows_tok[k] = 0;
                fr.rows_out[k] = k;
                *fr.n_items = base + kept;
            }
        }
        const int rk = item - base;
        if (rk < kept) {
            const uint64_t hit = __ballot(mine && below == rk);   // exactly one lane
            const int src = (int)__builtin_ctzll(hit);
            const int e = __builtin_amdgcn_readlane(r.my_idx, src);
            // expert e's pointer sits in lane e % 64, register e / 64 (both uniform)
            const void* pe = ptr[0];
#pragma unroll
            for (int i = 1; i < EPL; ++i) pe = (e >> 6) == i ? ptr[i] : pe;
            const uint64_t pb = (uint64_t)pe;
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)pb, e & 63);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(pb >> 32), e & 63);
            if (lane == 0) {
                pick->blob = (const uint8_t*)(((uint64_t)hi << 32) | lo);
                pick->begin = rk;
                pick->row0 = src;
                pick->ok = 1;
            }
        } else if (lane == 0) {
            pick->ok = 0;
        }
    }
    __syncthreads();
    if (!pick->ok) return false;
    it.blob = pick->blob;
    it.begin = pick->begin;
    it.count = 1;
    it.row0 = pick->row0;
    if (blockIdx.x == 0 && threadIdx.x == 0) fr.items[item] = it;
    return true;
}

// Resident waves per SIMD the register budget must allow: the decode grid
// (9 work items x 64 tiles x 2 matrices, 3 waves each) then fits on the chip
// in one round.
template <int NCH, int MTK, bool GS, bool W8>
constexpr int gateup_waves_per_eu() {
    return W8 ? (NCH == 1 && MTK == 1 ? 3 : 2) : NCH == 1 && MTK == 1 ? 4 : NCH == 1 && !GS ? 4 : NCH == 1 ? 3 : 2;
}

// MTK == 1: one token, 16-row tiles (twice the workgroups of 32-row tiles,
// half the registers each). MTK == 4: batches, 32-row tiles; each work item
// takes the body that fits its token count (1, 2, or chunks of 4), which
// keeps the per-wave batches of weight rows large for the many experts that
// see one or two tokens. Both read the activation planes once for the pair
// of matrices.
template <int W, int NCH, int MTK, bool GS, bool W8>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(gateup_waves_per_eu<NCH, MTK, GS, W8>(), 8)))
void gateup_kernel(
    const WorkItem* __restrict__ items, const int32_t* __restrict__ n_items,
    const int32_t* __restrict__ rows_tok, const int32_t* __restrict__ rows_out,
    const uint32_t* __restrict__ xplanes, const float* __restrict__ xscale,
    uint32_t* __restrict__ hplanes, float* __restrict__ hscale, int H, int I, BlobLayout L,
    FusedRoute fr, ReadLog rl) {
    __shared__ float red[W * kBlock * (MTK == 1 ? 1 : 2 * 4)];
    __shared__ FusedPick pick;
    const int item = blockIdx.y;
    WorkItem it;
    if (MTK == 1 && fr.codes) {
        if (!fused_item(fr, item, it, &pick)) return;
    } else {
        if (item >= *n_items) return;
        it = items[item];
    }
    const int t = blockIdx.x;
    if constexpr (MTK == 1) {
        gateup_body<W, NCH, 1, GS, true, W8>(it, t, rows_tok, rows_out, xplanes, xscale, hplanes, hscale, H, I, L, red);
        log_read(rl, it.blob, 0, t, 16, 1);
    } else {
        log_read(rl, it.blob, 0, t, 32, it.count <= 2 ? 1 : (it.count + 3) / 4);
        if (it.count == 1)
            gateup_body<W, NCH, 1, GS, false, W8>(it, t, rows_tok, rows_out, xplanes, xscale, hplanes, hscale, H, I, L, red);
        else if (it.count == 2)
            gateup_body<W, NCH, 2, GS, false, W8>(it, t, rows_tok, rows_out, xplanes, xscale, hplanes, hscale, H, I, L, red);
        else
            gateup_body<W, NCH, 4, GS, false, W8>(it, t, rows_tok, rows_out, xplanes, xscale, hplanes, hscale, H, I, L, red);
    }
}

template <int W, int NCH, int MTK, bool GS>
void launch_t(dim3 grid, hipStream_t s, const WorkItem* items, const int32_t* n_items,
              const int32_t* rows_tok, const int32_t* rows_out, const uint32_t* xp,
              const float* xs, uint32_t* hp, float* hs, int H, int I, const BlobLayout& L,
              const FusedRoute& fr, const ReadLog& rl) {
    if (L.wbits == 8) {
        launch((gateup_kernel<W, NCH, MTK, GS, true>), grid, dim3(64 * W), 0, s, items, n_items,
               rows_tok, rows_out, xp, xs, hp, hs, H, I, L, fr, rl);
        return;
    }
    launch((gateup_kernel<W, NCH, MTK, GS, false>), grid, dim3(64 * W), 0, s, items, n_items,
                       rows_tok, rows_out, xp, xs, hp, hs, H, I, L, fr, rl);
}

template <int W, int NCH, bool GS>
void by_mt(int mt, dim3 grid, hipStream_t s, const WorkItem* items, const int32_t* n_items,
           const int32_t* rows_tok, const int32_t* rows_out, const uint32_t* xp, const float* xs,
           uint32_t* hp, float* hs, int H, int I, const BlobLayout& L, const FusedRoute& fr,
           const ReadLog& rl) {
    if (mt == 1) launch_t<W, NCH, 1, GS>(grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L, fr, rl);
    else launch_t<W, NCH, 4, GS>(grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L, fr, rl);
}

template <bool GS>
bool by_width(int C, int mt, dim3 grid, hipStream_t s, const WorkItem* items,
              const int32_t* n_items, const int32_t* rows_tok, const int32_t* rows_out,
              const uint32_t* xp, const float* xs, uint32_t* hp, float* hs, int H, int I,
              const BlobLayout& L, const FusedRoute& fr, const ReadLog& rl) {
    if (C <= 64) by_mt<1, 1, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L, fr, rl);
    else if (C <= 128) by_mt<2, 1, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L, fr, rl);
    else if (C <= 192) by_mt<3, 1, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L, fr, rl);
    else if (C <= 256) by_mt<4, 1, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L, fr, rl);
    else if (C <= 512) by_mt<4, 2, GS>(mt, grid, s, items, n_items, rows_tok, rows_out, xp, xs, hp, hs, H, I, L, fr, rl);
    else return false;
    return true;
}

}  // namespace

bool dispatch_gateup(int mt, int group, dim3 grid, hipStream_t s, const WorkItem* items,
                     const int32_t* n_items, const int32_t* rows_tok, const int32_t* rows_out,
                     const uint32_t* xplanes, const float* xscale, uint32_t* hplanes,
                     float* hscale, int H, int I, const BlobLayout& L, const FusedRoute& fr,
                     const ReadLog& rl) {
    const int C = H / kBlock;
    return group ? by_width<true>(C, mt, grid, s, items, n_items, rows_tok, rows_out, xplanes,
                                  xscale, hplanes, hscale, H, I, L, fr, rl)
                 : by_width<false>(C, mt, grid, s, items, n_items, rows_tok, rows_out, xplanes,
                                   xscale, hplanes, hscale, H, I, L, fr, rl);
}

}  // namespace coli
