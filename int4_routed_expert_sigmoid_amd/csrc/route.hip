// Router: logits (f32 router weights, double accumulation) and the fused
// sigmoid / selection-bias / top-k / normalise step.
//
// lbrq.cn article "github一周涨11k⭐️！25GB 内存跑 744B GLM-5.2 模型！",
// section 三 item 1: a DeepSeek-V3-style sigmoid router picks 8 of 256
// experts per token; section 四 item 3: the aux-loss-free balancing bias
// adjusts the selection, and routing, selection and scaling semantics must be
// reproduced exactly. config.json values quoted by the int8-MTP page:
// scoring_func sigmoid, norm_topk_prob true.
#include <algorithm>

#include "common.h"

namespace coli {
namespace {

// One wave per (token, expert): lanes stride the hidden axis with double
// FMAs; the wave sum is rounded once to float.
__global__ __launch_bounds__(256) void logits_kernel(const float* __restrict__ wr,
                                                     const float* __restrict__ x, int T, int H,
                                                     int E, float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= (int64_t)T * E) return;
    const int t = (int)(pair / E), e = (int)(pair % E);
    const float* wrow = wr + (int64_t)e * H;
    const float* xrow = x + (int64_t)t * H;
    double acc = 0.0;
    for (int j = lane; j < H; j += 64) acc = fma((double)wrow[j], (double)xrow[j], acc);
    acc = wave_sum_f64(acc);
    if (lane == 0) logits[pair] = (float)acc;
}

constexpr int kMaxExpertsPerLane = 16;   // E <= 1024

// Route one token with one wave (the selection helpers are in common.h).
// Lane l holds experts l, l+64, ...; all loads first (clamped ids), then
// branch-free arithmetic.
template <int EPL>
__device__ __forceinline__ void route_token(const float* __restrict__ lrow,
                                            const float* __restrict__ bias, int E, int k,
                                            float topp, int* __restrict__ idx_row,
                                            float* __restrict__ w_row, int* lds_idx = nullptr) {
    const int lane = threadIdx.x & 63;
    uint64_t code[EPL];
    float score[EPL], lv[EPL], bv[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = min(lane + 64 * i, E - 1);
        lv[i] = lrow[e];
        bv[i] = bias ? bias[e] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        const bool valid = e < E;
        const float s = sigmoid_score(lv[i]);
        score[i] = valid ? s : 0.f;
        code[i] = valid ? selection_code(s + bv[i], e) : 0;
    }
    const TopK r = select_topk<EPL>(code, score, k, topp);
    if (lane < k) {
        const bool kp = lane < r.kept;
        idx_row[lane] = kp ? r.my_idx : -1;
        w_row[lane] = kp ? r.my_w : 0.f;
        if (lds_idx) lds_idx[lane] = kp ? r.my_idx : -1;
    }
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int k, float topp, int* __restrict__ idx,
                                                    float* __restrict__ w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    route_token<EPL>(logits + (int64_t)t * E, bias, E, k, topp, idx + (int64_t)t * k,
                     w + (int64_t)t * k);
}

// ----------------------------------------------------- router, small T
// Two launches for batches of up to kSmallT tokens. The first spreads over
// many workgroups: one per expert computes its logits (f32 router rows,
// double sums), the others encode the activations into digit planes.
// The second is one workgroup: it routes the tokens, forms the batch union
// (stable counting sort) and writes the FFN work list.
constexpr int kRouterThreads = 256;

__device__ __forceinline__ double block_sum_f64(double v, double* sh) {
    v = wave_sum_f64(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    return sh[0] + sh[1] + sh[2] + sh[3];
}

// Workgroups [0, NR) (NR = E when there are router rows or selection codes to
// write, else 0): one expert's logits for every token, then, for one token
// with the routing folded into the gate/up pass, its score and selection
// code. Workgroups from NR on: the digit-plane encoding of x, one quarter
// block per thread.
__global__ __launch_bounds__(kRouterThreads) void router_prep_kernel(SmallRouterArgs a) {
    __shared__ double shd[4];
    const int tid = threadIdx.x;
    const int T = a.T, E = a.E, H = a.H;
    const int NR = a.router_w || a.codes ? E : 0;
    if ((int)blockIdx.x < NR) {
        const int e = blockIdx.x;
        // the bias and given logit of this expert, requested before the row's loads
        const float bias_e = a.codes && a.bias ? a.bias[e] : 0.f;
        const float logit_in = a.codes && !a.router_w ? a.logits_in[e] : 0.f;
        float logit0 = 0.f;                         // token 0's logit (thread 0)
        if (a.router_w) {
            const float* wrow = a.router_w + (int64_t)e * H;
            constexpr int kStep = kRouterThreads * 4, kU = 8;   // floats per pass, passes per load group
            for (int t = 0; t < T; ++t) {
                const float* xrow = a.x + (int64_t)t * H;
                double acc = 0.0;
                // kU passes' loads in flight at once (clamped addresses, masked
                // values), then the f64 FMAs in column order
                for (int j0 = tid * 4; j0 < H; j0 += kU * kStep) {
                    float4 wv[kU], xv[kU];
#pragma unroll
                    for (int u = 0; u < kU; ++u) {
                        const int j = min(j0 + u * kStep, H - 4);
                        wv[u] = *reinterpret_cast<const float4*>(wrow + j);
                        xv[u] = *reinterpret_cast<const float4*>(xrow + j);
                    }
#pragma unroll
                    for (int u = 0; u < kU; ++u) {
                        if (j0 + u * kStep < H) {
                            acc = fma((double)wv[u].x, (double)xv[u].x, acc);
                            acc = fma((double)wv[u].y, (double)xv[u].y, acc);
                            acc = fma((double)wv[u].z, (double)xv[u].z, acc);
                            acc = fma((double)wv[u].w, (double)xv[u].w, acc);
                        }
                    }
                }
                acc = block_sum_f64(acc, shd);
                if (tid == 0) {
                    a.logits_out[(int64_t)t * E + e] = (float)acc;
                    if (t == 0) logit0 = (float)acc;
                }
            }
        }
        if (a.codes && tid == 0) {
            const float s = sigmoid_score(a.router_w ? logit0 : logit_in);
            a.scores[e] = s;
            a.codes[e] = selection_code(s + bias_e, e);
        }
        return;
    }
    const int C = H / kBlock;
    const int64_t g = (int64_t)(blockIdx.x - NR) * kRouterThreads + tid;
    const int q = (int)(g & 3);
    const int64_t blk = g >> 2;
    const int64_t row = blk / C;
    const int b = (int)(blk % C);
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const bool ok = row < T;
    if (ok) {
        const float* p = a.x + row * H + b * kBlock + q * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = p[i];
    }
    uint32_t words[kPlanes];
    const float sc = encode_quarter(v, words);
    if (ok) {
        uint32_t* out = a.xplanes + (row * C + b) * kWordsPerBlock;
#pragma unroll
        for (int p = 0; p < kPlanes; ++p) out[p * 4 + q] = words[p];
        if (q == 0) a.xscale[row * C + b] = sc;
    }
}

// Exclusive prefix sum over the 256 threads of the block, modulo 2^32;
// *total receives the sum. Wave scans by shuffles, then one pass over the
// wave totals.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) sh[wave] = incl;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wave; ++w) base += sh[w];
    *total = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();
    return base + incl - v;
}

template <int EPL>
__global__ __launch_bounds__(kRouterThreads) void router_plan_kernel(SmallRouterArgs a) {
    constexpr int EPT = 4;                  // experts per thread (E <= 1024)
    __shared__ int s_idx[kSmallT * 32];
    __shared__ int s_cnt[1024];
    __shared__ int s_off[1024];
    __shared__ int s_first[1024];
    __shared__ uint32_t s_scan[4];
    const int tid = threadIdx.x, wave = tid >> 6;
    const int T = a.T, E = a.E, k = a.k;
    const float* lg = a.router_w ? a.logits_out : a.logits_in;
    // blob pointers of this thread's experts, loaded now so that their latency
    // hides behind the routing
    const bool with_items = a.table != nullptr;
    const void* tptr[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        tptr[i] = (with_items && e < E) ? a.table[e] : nullptr;
    }
    for (int t = wave; t < T; t += kRouterThreads / 64)
        route_token<EPL>(lg + (int64_t)t * E, a.bias, E, k, a.topp, a.idx + (int64_t)t * k,
                         a.w + (int64_t)t * k, s_idx + t * k);
    const int base = a.shared_blob ? 1 : 0;
    // the shared expert's items (its T tokens, split like the routed experts')
    const int sbase = !a.shared_blob ? 0 : a.split ? (T + kItemTokens - 1) / kItemTokens : 1;
    if (T == 1 && a.phase_mask == nullptr) {
        // one token: the k picks are distinct, so the union is their order by
        // expert id; every count is 0 or 1 and each offset is the number of
        // picks below the expert
        __syncthreads();
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid * EPT + i;
            if (e < E) {
                // dropped slots hold -1, which is above every id as unsigned
                int c = 0, below = 0, slot = 0;
                for (int j = 0; j < k; ++j) {
                    c += s_idx[j] == e;
                    slot = s_idx[j] == e ? j : slot;
                    below += (uint32_t)s_idx[j] < (uint32_t)e;
                }
                a.counts[e] = c;
                a.offsets[e] = below;
                if (c) {
                    a.unique[below] = e;
                    if (with_items) {
                        WorkItem it;
                        it.blob = (const uint8_t*)tptr[i];
                        it.begin = below;
                        it.count = 1;
                        it.row0 = slot;
                        a.items[base + below] = it;
                    }
                }
            }
        }
        int kept = 0;
        for (int j = 0; j < k; ++j) kept += s_idx[j] >= 0;
        if (tid < k && s_idx[tid] >= 0) {
            const int e = s_idx[tid];
            int p = 0;
            for (int j = 0; j < k; ++j) p += (uint32_t)s_idx[j] < (uint32_t)e;
            a.perm[p] = tid;
            a.rows_tok[p] = 0;
            a.rows_out[p] = tid;
        }
        if (tid == 0) {
            a.offsets[E] = kept;
            *a.n_unique = kept;
            a.rows_tok[k] = 0;
            a.rows_out[k] = k;
            if (with_items && a.shared_blob) {
                WorkItem it;
                it.blob = (const uint8_t*)a.shared_blob;
                it.begin = k;
                it.count = 1;
                it.row0 = k;
                a.items[0] = it;
            }
            *a.n_items = with_items ? base + kept : 0;
        }
        return;
    }
    for (int e = tid; e < E; e += kRouterThreads) {
        s_cnt[e] = 0;
        s_first[e] = 0x7fffffff;
    }
    __syncthreads();
    // batch union of the n = T*k assignments (stable counting sort)
    const int n = T * k;
    for (int i = tid; i < n; i += kRouterThreads) {
        const int e = s_idx[i];
        if (e < 0) continue;                        // dropped by top-p
        atomicAdd(&s_cnt[e], 1);
        atomicMin(&s_first[e], i);                  // an item's first row is its first assignment
    }
    __syncthreads();
    // offsets, the unique list and the kept work items in one scan: thread
    // tid owns experts tid*EPT .. tid*EPT+3 and scans the packed triple
    // (assignments << 22 | unique << 11 | work items); the fields cannot carry
    // (assignments and items <= 512, experts <= 1024)
    int c[EPT];
    uint32_t packed = 0;
    int nit[EPT];                           // work items of the expert (0: not kept)
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        c[i] = e < E ? s_cnt[e] : 0;
        const bool keep = with_items && c[i] > 0 &&
                          (a.phase_mask == nullptr || a.phase_mask[e] == a.phase);
        nit[i] = !keep ? 0 : a.split ? (c[i] + kItemTokens - 1) / kItemTokens : 1;
        packed += ((uint32_t)c[i] << 22) + ((uint32_t)(c[i] > 0) << 11) + (uint32_t)nit[i];
    }
    uint32_t total = 0;
    const uint32_t pre = block_excl_scan(packed, s_scan, &total);
    int off = (int)(pre >> 22), upos = (int)((pre >> 11) & 0x7FF), kpos = (int)(pre & 0x7FF);
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        if (e < E) {
            a.counts[e] = c[i];
            a.offsets[e] = off;
            s_off[e] = off;
            if (c[i] > 0) a.unique[upos++] = e;
            for (int p = 0; p < nit[i]; ++p) {
                const int first = a.split ? p * kItemTokens : 0;
                WorkItem it;
                it.blob = (const uint8_t*)tptr[i];
                it.begin = off + first;
                it.count = a.split ? min(kItemTokens, c[i] - first) : c[i];
                it.row0 = s_first[e];
                a.items[sbase + kpos++] = it;
            }
            off += c[i];
        }
    }
    if (tid == 0) {
        a.offsets[E] = (int)(total >> 22);
        *a.n_unique = (int)((total >> 11) & 0x7FF);
        // work items: the shared expert first, then the kept unique experts;
        // without a table (cached calls) the items are formed later
        if (with_items && a.shared_blob) {
            for (int p = 0; p < sbase; ++p) {
                const int first = a.split ? p * kItemTokens : 0;
                WorkItem it;
                it.blob = (const uint8_t*)a.shared_blob;
                it.begin = n + first;
                it.count = a.split ? min(kItemTokens, T - first) : T;
                it.row0 = n + first;
                a.items[p] = it;
            }
        }
        *a.n_items = with_items ? sbase + (int)(total & 0x7FF) : 0;
    }
    __syncthreads();
    // stable positions: rank of assignment i among earlier equal experts
    for (int i = tid; i < n; i += kRouterThreads) {
        const int e = s_idx[i];
        if (e < 0) continue;
        int r = 0;
        for (int j = 0; j < i; ++j) r += (s_idx[j] == e) ? 1 : 0;
        const int p = s_off[e] + r;
        a.perm[p] = i;
        a.rows_tok[p] = i / k;
        a.rows_out[p] = i;
    }
    for (int t = tid; t < T; t += kRouterThreads) {
        a.rows_tok[n + t] = t;
        a.rows_out[n + t] = n + t;
    }
}

}  // namespace

coli_status launch_router_logits(const float* wr, const float* x, int32_t T, int32_t H, int32_t E,
                                 float* logits, hipStream_t stream) {
    const int64_t pairs = (int64_t)T * E;
    if (pairs == 0) return COLI_OK;
    launch(logits_kernel, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, stream, wr,
                       x, T, H, E, logits);
    COLI_CHECK_LAUNCH("router logits kernel launch");
    return COLI_OK;
}

coli_status launch_router_small(const SmallRouterArgs& a, hipStream_t stream) {
    const int C = a.H / kBlock;
    const int enc_blocks = (int)(((int64_t)a.T * C * 4 + kRouterThreads - 1) / kRouterThreads);
    const int grid = (a.router_w || a.codes ? a.E : 0) + enc_blocks;
    launch(router_prep_kernel, dim3(grid), dim3(kRouterThreads), 0, stream, a);
    COLI_CHECK_LAUNCH("router prep kernel launch");
    if (a.codes) return COLI_OK;        // the gate/up pass routes (FusedRoute)
    const int epl = (a.E + 63) / 64;
    const dim3 one(1), blk(kRouterThreads);
    if (epl <= 1) launch(router_plan_kernel<1>, one, blk, 0, stream, a);
    else if (epl <= 2) launch(router_plan_kernel<2>, one, blk, 0, stream, a);
    else if (epl <= 4) launch(router_plan_kernel<4>, one, blk, 0, stream, a);
    else if (epl <= 8) launch(router_plan_kernel<8>, one, blk, 0, stream, a);
    else launch(router_plan_kernel<16>, one, blk, 0, stream, a);
    COLI_CHECK_LAUNCH("router plan kernel launch");
    return COLI_OK;
}

coli_status launch_route(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                         float topp, int32_t* idx, float* w, hipStream_t stream) {
    if (T == 0) return COLI_OK;
    const dim3 grid((T + 3) / 4), block(256);
    const int epl = (E + 63) / 64;
    if (epl <= 1) launch(route_kernel<1>, grid, block, 0, stream, logits, bias, T, E, k, topp, idx, w);
    else if (epl <= 2) launch(route_kernel<2>, grid, block, 0, stream, logits, bias, T, E, k, topp, idx, w);
    else if (epl <= 4) launch(route_kernel<4>, grid, block, 0, stream, logits, bias, T, E, k, topp, idx, w);
    else if (epl <= 8) launch(route_kernel<8>, grid, block, 0, stream, logits, bias, T, E, k, topp, idx, w);
    else if (epl <= kMaxExpertsPerLane) launch(route_kernel<16>, grid, block, 0, stream, logits, bias, T, E, k, topp, idx, w);
    else return fail(COLI_EUNSUPPORTED, "route: more than 1024 experts");
    COLI_CHECK_LAUNCH("route kernel launch");
    return COLI_OK;
}

}  // namespace coli
