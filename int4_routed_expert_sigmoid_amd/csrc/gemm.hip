// Prefill / large-batch expert FFN on bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Batch union (lbrq.cn article section 三 item 4; practical guide section 二):
// every unique expert's weights are applied to all of its tokens as one
// grouped GEMM: h = silu(Xe Wg^T) * (Xe Wu^T), ye = h Wd^T, where Xe holds the
// rows of the expert's tokens. Tiles of 64 tokens x 64 rows (x gate and up)
// or 64 tokens x 128 rows (down); a device-built list of 64-token tiles per
// work item lets one launch cover every expert whatever its token count.
//
// Operands. A (activations) is bf16: x rounded once to bf16 by a prep pass,
// h rounded to bf16 in the gate/up epilogue. B (weights) is the int4 code
// plus 136, which is exact in bf16 (values 128..143): the unsigned nibble
// u = q + 8 placed in the mantissa of 128.0 with two byte permutes. Hence
//   sum_k (136 + q_k) a_k = sum_k q_k a_k + 136 * S,  S = sum_k a_k,
// and each output subtracts 136 * S, where S sums the same bf16 values in a
// fixed order (per 64-column group, which also serves gs64 scales). The
// per-row or per-group f32 scale is applied after the MFMA sum.
//
// MFMA operand layout used here (32x32x16): lane l supplies A[m][k] and
// B[k][n] for m = n = l % 32 and the 8 k-values of half l / 32. K-step s of a
// 64-wide k block maps half h, element j to k = 32h + 8s + j, so one 16-byte
// load per lane covers 32 consecutive k of one weight row (4 K-steps) and
// 64 bytes of its activation row. Accumulator element j of lane l is
// C[8(j/4) + 4(l/32) + j%4][l % 32].
#include <algorithm>

#include "common.h"
#include "gemm.h"

namespace coli {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;

constexpr int kTileM = 64;
constexpr float kOffset = 136.0f;   // bf16 B operand = q + 136

__device__ __forceinline__ uint4 ldg16(const void* p) {
    const u32x4 v = *(g_u32x4*)(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 8 nibbles (two's complement, column order) -> 8 bf16 values q + 136 in
// MFMA operand order (element j <-> column j).
__device__ __forceinline__ bf16x8 nib8_to_bf16(uint32_t w) {
    const uint32_t u = w ^ 0x88888888u;                 // q + 8 in every nibble
    const uint32_t lo = u & 0x0F0F0F0Fu;                // columns 0, 2, 4, 6
    const uint32_t hi = (u >> 4) & 0x0F0F0F0Fu;         // columns 1, 3, 5, 7
    const uint32_t p01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);   // u0 u1 u2 u3
    const uint32_t p23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);   // u4 u5 u6 u7
    uint4 r;
    r.x = __builtin_amdgcn_perm(0x43434343u, p01, 0x05010400u);        // 128+u0, 128+u1
    r.y = __builtin_amdgcn_perm(0x43434343u, p01, 0x05030402u);
    r.z = __builtin_amdgcn_perm(0x43434343u, p23, 0x05010400u);
    r.w = __builtin_amdgcn_perm(0x43434343u, p23, 0x05030402u);
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float bf16_round(float f) {
    return (float)(__bf16)f;
}

__device__ __forceinline__ uint16_t bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// ---------------------------------------------------------------- prep
// x [T][H] f32 -> xb [T][H] bf16 and S_x [T][H/64] (sums of the bf16 values of
// each 64-column group, left to right). One thread per group.
__global__ __launch_bounds__(256) void prep_kernel(const float* __restrict__ x, int T, int H,
                                                   uint16_t* __restrict__ xb,
                                                   float* __restrict__ sx) {
    const int G = H / 64;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (int64_t)T * G) return;
    const int64_t t = gid / G;
    const int g = (int)(gid % G);
    const float* src = x + t * H + g * 64;
    uint16_t* dst = xb + t * H + g * 64;
    float s = 0.f;
    for (int j = 0; j < 64; j += 8) {
        const float4 a = *reinterpret_cast<const float4*>(src + j);
        const float4 b = *reinterpret_cast<const float4*>(src + j + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint16_t l = bf16_bits(v[2 * i]), h = bf16_bits(v[2 * i + 1]);
            pk[i] = (uint32_t)l | ((uint32_t)h << 16);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) s += bf16_round(v[i]);
        *reinterpret_cast<uint4*>(dst + j) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    }
    sx[t * G + g] = s;
}

// ------------------------------------------------------------ tile list
// (item, first token) of every 64-token tile, items in order.
__global__ __launch_bounds__(256) void tiles_kernel(const WorkItem* __restrict__ items,
                                                    const int32_t* __restrict__ n_items,
                                                    int2* __restrict__ tiles,
                                                    int32_t* __restrict__ n_tiles) {
    __shared__ int sh[256];
    const int t = threadIdx.x;
    const int ni = *n_items;
    int base = 0;
    for (int i0 = 0; i0 < ni; i0 += 256) {
        const int i = i0 + t;
        const int c = i < ni ? (items[i].count + kTileM - 1) / kTileM : 0;
        sh[t] = c;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            const int add = t >= o ? sh[t - o] : 0;
            __syncthreads();
            sh[t] += add;
            __syncthreads();
        }
        const int start = base + sh[t] - c;
        for (int j = 0; j < c; ++j) tiles[start + j] = make_int2(i, j * kTileM);
        base += sh[255];
        __syncthreads();
    }
    if (t == 0) *n_tiles = base;
}

// ----------------------------------------------------------------- gate/up
// Workgroup: 64 tokens of one item x 64 intermediate rows of gate and up.
// Wave (wm, wi): tokens 32wm.., rows 32wi.., one 32x32 accumulator per matrix.
template <bool GS>
__global__ __launch_bounds__(256) void gemm_gateup_kernel(GemmArgs a) {
    __shared__ float s_part[2][kTileM];          // per-wave row sums of bf16(h)
    __shared__ float s_tot[kTileM];              // per-token sum of the bf16 x row
    const int tile = blockIdx.x;
    if (tile >= *a.n_tiles) return;
    const int2 td = a.tiles[tile];
    const WorkItem it = a.items[td.x];
    const int m0 = td.y;
    if (!GS && threadIdx.x < kTileM) {
        const int tok = a.rows_tok[it.begin + min(m0 + (int)threadIdx.x, it.count - 1)];
        const int G = a.H / 64;
        float s = 0.f;
        for (int q = 0; q < G; ++q) s += a.sx[(size_t)tok * G + q];
        s_tot[threadIdx.x] = s;
    }
    __syncthreads();
    const int nt = blockIdx.y;                   // 64-row block of the intermediate axis
    const int H = a.H, I = a.I;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wi = wave >> 1;
    const int ln = lane & 31, lh = lane >> 5;
    const BlobLayout& L = a.L;
    const uint8_t* gq = it.blob + L.gate_q;
    const uint8_t* uq = it.blob + L.up_q;
    const float* gsc = reinterpret_cast<const float*>(it.blob + L.gate_s);
    const float* usc = reinterpret_cast<const float*>(it.blob + L.up_s);
    const int G = H / 64;

    // this lane's A row (token) and B rows (intermediate index)
    const int pm = m0 + wm * 32 + ln;                        // token position in the item
    const int arow = a.rows_tok[it.begin + min(pm, it.count - 1)];
    const uint16_t* ap = a.xb + (size_t)arow * H + lh * 32;
    const int irow = nt * 64 + wi * 32 + ln;
    const uint8_t* gp = gq + (size_t)irow * (H / 2) + lh * 16;
    const uint8_t* up = uq + (size_t)irow * (H / 2) + lh * 16;

    f32x16 accg = {}, accu = {};
    f32x16 totg = {}, totu = {};                 // gs64: scaled sum over groups
    uint4 A[4], Bg, Bu, An[4], Bgn, Bun;
#pragma unroll
    for (int s = 0; s < 4; ++s) A[s] = ldg16(ap + 8 * s);
    Bg = ldg16(gp);
    Bu = ldg16(up);
    for (int kb = 0; kb < G; ++kb) {
        const bool more = kb + 1 < G;
        if (more) {
#pragma unroll
            for (int s = 0; s < 4; ++s) An[s] = ldg16(ap + (kb + 1) * 64 + 8 * s);
            Bgn = ldg16(gp + (kb + 1) * 32);
            Bun = ldg16(up + (kb + 1) * 32);
        }
        const uint32_t wg[4] = {Bg.x, Bg.y, Bg.z, Bg.w};
        const uint32_t wu[4] = {Bu.x, Bu.y, Bu.z, Bu.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bf16x8 av = as_bf16x8(A[s]);
            accg = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, nib8_to_bf16(wg[s]), accg, 0, 0, 0);
            accu = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, nib8_to_bf16(wu[s]), accu, 0, 0, 0);
        }
        if (GS) {
            // one 64-column group per k block: scale it and start a new sum
            const float fg = gsc[(size_t)irow * G + kb], fu = usc[(size_t)irow * G + kb];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int m = m0 + wm * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);
                const int tok = a.rows_tok[it.begin + min(m, it.count - 1)];
                const float cs = kOffset * a.sx[(size_t)tok * G + kb];
                totg[j] = fmaf(fg, accg[j] - cs, totg[j]);
                totu[j] = fmaf(fu, accu[j] - cs, totu[j]);
                accg[j] = 0.f;
                accu[j] = 0.f;
            }
        }
        if (more) {
#pragma unroll
            for (int s = 0; s < 4; ++s) A[s] = An[s];
            Bg = Bgn;
            Bu = Bun;
        }
    }
    // epilogue: h = silu(g) * u -> bf16, and per-token sums of the bf16 h
    const float fg = GS ? 1.f : gsc[irow], fu = GS ? 1.f : usc[irow];
    float rsum[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int m = m0 + wm * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);
        float g, u;
        if (GS) {
            g = totg[j];
            u = totu[j];
        } else {
            const float sxt = s_tot[m - m0 < kTileM ? m - m0 : 0];
            g = fg * (accg[j] - kOffset * sxt);
            u = fu * (accu[j] - kOffset * sxt);
        }
        const float h = g / (1.f + expf(-g)) * u;
        const uint16_t hb = bf16_bits(h);
        rsum[j] = bf16_round(h);
        if (m < it.count) {
            const int out = a.rows_out[it.begin + m];
            a.hb[(size_t)out * I + irow] = hb;
        }
    }
    // sum over the 32 rows of this wave (lanes sharing lh), fixed butterfly order
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        float v = rsum[j];
        v += __int_as_float(lane_xchg<1>(__float_as_int(v)));
        v += __int_as_float(lane_xchg<2>(__float_as_int(v)));
        v += __int_as_float(lane_xchg<4>(__float_as_int(v)));
        v += __int_as_float(lane_xchg<8>(__float_as_int(v)));
        v += __int_as_float(lane_xchg<16>(__float_as_int(v)));
        rsum[j] = v;
    }
    if (ln == 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) s_part[wi][wm * 32 + 8 * (j >> 2) + 4 * lh + (j & 3)] = rsum[j];
    }
    __syncthreads();
    if (threadIdx.x < kTileM) {
        const int m = m0 + threadIdx.x;
        if (m < it.count) {
            const int out = a.rows_out[it.begin + m];
            a.sh[(size_t)out * (I / 64) + nt] = s_part[0][threadIdx.x] + s_part[1][threadIdx.x];
        }
    }
}

// -------------------------------------------------------------------- down
// Workgroup: 64 tokens of one item x 128 output columns. Wave (wm, wn):
// tokens 32wm.., columns 64wn.. (two 32x32 accumulators).
template <bool GS>
__global__ __launch_bounds__(256) void gemm_down_kernel(GemmArgs a) {
    __shared__ float s_tot[kTileM];              // per-row sum of the bf16 h row
    const int tile = blockIdx.x;
    if (tile >= *a.n_tiles) return;
    const int2 td = a.tiles[tile];
    const WorkItem it = a.items[td.x];
    const int m0 = td.y;
    if (!GS && threadIdx.x < kTileM) {
        const int out = a.rows_out[it.begin + min(m0 + (int)threadIdx.x, it.count - 1)];
        const int GI = a.I / 64;
        float s = 0.f;
        for (int q = 0; q < GI; ++q) s += a.sh[(size_t)out * GI + q];
        s_tot[threadIdx.x] = s;
    }
    __syncthreads();
    const int H = a.H, I = a.I;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int ln = lane & 31, lh = lane >> 5;
    const BlobLayout& L = a.L;
    const uint8_t* dq = it.blob + L.down_q;
    const float* dsc = reinterpret_cast<const float*>(it.blob + L.down_s);
    const int GI = I / 64;

    const int pm = m0 + wm * 32 + ln;
    const int arow = a.rows_out[it.begin + min(pm, it.count - 1)];
    const uint16_t* ap = a.hb + (size_t)arow * I + lh * 32;
    const int c0 = blockIdx.y * 128 + wn * 64 + ln;          // first of this lane's 2 columns
    const uint8_t* bp0 = dq + (size_t)min(c0, H - 1) * (I / 2) + lh * 16;
    const uint8_t* bp1 = dq + (size_t)min(c0 + 32, H - 1) * (I / 2) + lh * 16;

    f32x16 acc0 = {}, acc1 = {}, tot0 = {}, tot1 = {};
    uint4 A[4], B0, B1, An[4], B0n, B1n;
#pragma unroll
    for (int s = 0; s < 4; ++s) A[s] = ldg16(ap + 8 * s);
    B0 = ldg16(bp0);
    B1 = ldg16(bp1);
    for (int kb = 0; kb < GI; ++kb) {
        const bool more = kb + 1 < GI;
        if (more) {
#pragma unroll
            for (int s = 0; s < 4; ++s) An[s] = ldg16(ap + (kb + 1) * 64 + 8 * s);
            B0n = ldg16(bp0 + (kb + 1) * 32);
            B1n = ldg16(bp1 + (kb + 1) * 32);
        }
        const uint32_t w0[4] = {B0.x, B0.y, B0.z, B0.w};
        const uint32_t w1[4] = {B1.x, B1.y, B1.z, B1.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bf16x8 av = as_bf16x8(A[s]);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, nib8_to_bf16(w0[s]), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, nib8_to_bf16(w1[s]), acc1, 0, 0, 0);
        }
        if (GS) {
            const float f0 = dsc[(size_t)min(c0, H - 1) * GI + kb];
            const float f1 = dsc[(size_t)min(c0 + 32, H - 1) * GI + kb];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int m = m0 + wm * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);
                const int out = a.rows_out[it.begin + min(m, it.count - 1)];
                const float cs = kOffset * a.sh[(size_t)out * GI + kb];
                tot0[j] = fmaf(f0, acc0[j] - cs, tot0[j]);
                tot1[j] = fmaf(f1, acc1[j] - cs, tot1[j]);
                acc0[j] = 0.f;
                acc1[j] = 0.f;
            }
        }
        if (more) {
#pragma unroll
            for (int s = 0; s < 4; ++s) A[s] = An[s];
            B0 = B0n;
            B1 = B1n;
        }
    }
    const float f0 = GS ? 1.f : dsc[min(c0, H - 1)], f1 = GS ? 1.f : dsc[min(c0 + 32, H - 1)];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int m = m0 + wm * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);
        if (m >= it.count) continue;
        const int out = a.rows_out[it.begin + m];
        float y0, y1;
        if (GS) {
            y0 = tot0[j];
            y1 = tot1[j];
        } else {
            const float s = s_tot[m - m0];
            y0 = f0 * (acc0[j] - kOffset * s);
            y1 = f1 * (acc1[j] - kOffset * s);
        }
        if (c0 < H) a.y_rows[(size_t)out * H + c0] = y0;
        if (c0 + 32 < H) a.y_rows[(size_t)out * H + c0 + 32] = y1;
    }
}

}  // namespace

size_t gemm_tiles_max(int32_t rows, int32_t max_items) {
    return (size_t)rows / kTileM + (size_t)max_items + 1;
}

coli_status launch_mfma_ffn(const GemmArgs& a, const float* x, int32_t T, int32_t max_tiles,
                            hipStream_t stream) {
    if (a.H % 64 || a.I % 64) return fail(COLI_EUNSUPPORTED, "mfma path: hidden and inter must be multiples of 64");
    const int G = a.H / 64;
    const int64_t prep_threads = (int64_t)T * G;
    launch(prep_kernel, dim3((unsigned)((prep_threads + 255) / 256)), dim3(256), 0, stream, x, T,
           a.H, a.xb, a.sx);
    COLI_CHECK_LAUNCH("prep kernel launch");
    launch(tiles_kernel, dim3(1), dim3(256), 0, stream, a.items, a.n_items, a.tiles, a.n_tiles);
    COLI_CHECK_LAUNCH("tile list kernel launch");
    {
        ProfTag prof("gemm_gateup");
        const dim3 grid(max_tiles, a.I / 64);
        if (a.group) launch(gemm_gateup_kernel<true>, grid, dim3(256), 0, stream, a);
        else launch(gemm_gateup_kernel<false>, grid, dim3(256), 0, stream, a);
    }
    COLI_CHECK_LAUNCH("gate/up GEMM launch");
    {
        ProfTag prof("gemm_down");
        const dim3 grid(max_tiles, (a.H + 127) / 128);
        if (a.group) launch(gemm_down_kernel<true>, grid, dim3(256), 0, stream, a);
        else launch(gemm_down_kernel<false>, grid, dim3(256), 0, stream, a);
    }
    COLI_CHECK_LAUNCH("down GEMM launch");
    return COLI_OK;
}

}  // namespace coli
