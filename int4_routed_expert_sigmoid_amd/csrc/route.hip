// Router: logits (f32 router weights, double accumulation) and the fused
// sigmoid / selection-bias / top-k / normalise step.
//
// lbrq.cn article "github一周涨11k⭐️！25GB 内存跑 744B GLM-5.2 模型！",
// section 三 item 1: a DeepSeek-V3-style sigmoid router picks 8 of 256
// experts per token; section 四 item 3: the aux-loss-free balancing bias
// adjusts the selection, and routing, selection and scaling semantics must be
// reproduced exactly. config.json values quoted by the int8-MTP page:
// scoring_func sigmoid, norm_topk_prob true.
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
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) logits[pair] = (float)acc;
}

constexpr int kMaxExpertsPerLane = 16;   // E <= 1024

// One wave per token. Lane l holds experts l, l+64, ... . k rounds of a wave
// arg-max over (key descending, index ascending) pick the experts in slot
// order; the weights are normalised in double in slot order.
template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int k, int* __restrict__ idx,
                                                    float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    float score[EPL], key[EPL];
    bool avail[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        avail[i] = e < E;
        score[i] = 0.f;
        key[i] = 0.f;
        if (avail[i]) {
            const double l = (double)logits[(int64_t)t * E + e];
            score[i] = (float)(1.0 / (1.0 + exp(-l)));
            key[i] = score[i] + (bias ? bias[e] : 0.f);
        }
    }
    double sum = 0.0;
    float my_sel = 0.f;      // lane j (< k) keeps the score of slot j
    int my_idx = 0;
    for (int j = 0; j < k; ++j) {
        // best candidate of this lane
        float bk = 0.f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            if (!avail[i]) continue;
            const int e = lane + 64 * i;
            if (bi == 0x7fffffff || key[i] > bk) { bk = key[i]; bi = e; }
        }
        // wave arg-max: larger key wins, equal keys go to the lower index
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ok = __shfl_xor(bk, o);
            const int oi = __shfl_xor(bi, o);
            if (oi != 0x7fffffff && (bi == 0x7fffffff || ok > bk || (ok == bk && oi < bi))) {
                bk = ok;
                bi = oi;
            }
        }
        const int owner = bi & 63, slot = bi >> 6;
        float s_sel = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (i == slot && lane == owner) { avail[i] = false; s_sel = score[i]; }
        s_sel = __shfl(s_sel, owner);
        sum += (double)s_sel;
        if (lane == j) { my_sel = s_sel; my_idx = bi; }
    }
    if (lane < k) {
        idx[(int64_t)t * k + lane] = my_idx;
        w[(int64_t)t * k + lane] = (sum == 0.0) ? (float)(1.0 / k) : (float)((double)my_sel / sum);
    }
}

}  // namespace

coli_status launch_router_logits(const float* wr, const float* x, int32_t T, int32_t H, int32_t E,
                                 float* logits, hipStream_t stream) {
    const int64_t pairs = (int64_t)T * E;
    if (pairs == 0) return COLI_OK;
    hipLaunchKernelGGL(logits_kernel, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, stream, wr,
                       x, T, H, E, logits);
    COLI_CHECK_LAUNCH("router logits kernel launch");
    return COLI_OK;
}

coli_status launch_route(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                         int32_t* idx, float* w, hipStream_t stream) {
    if (T == 0) return COLI_OK;
    const dim3 grid((T + 3) / 4), block(256);
    const int epl = (E + 63) / 64;
    if (epl <= 1) hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, stream, logits, bias, T, E, k, idx, w);
    else if (epl <= 2) hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, stream, logits, bias, T, E, k, idx, w);
    else if (epl <= 4) hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, stream, logits, bias, T, E, k, idx, w);
    else if (epl <= 8) hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, stream, logits, bias, T, E, k, idx, w);
    else if (epl <= kMaxExpertsPerLane) hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, stream, logits, bias, T, E, k, idx, w);
    else return fail(COLI_EUNSUPPORTED, "route: more than 1024 experts");
    COLI_CHECK_LAUNCH("route kernel launch");
    return COLI_OK;
}

}  // namespace coli
