// Prefill / large-batch expert FFN on bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Batch union (lbrq.cn article section 三 item 4; practical guide section 二):
// every unique expert's weights are applied to all of its tokens as one
// grouped GEMM: h = silu(Xe Wg^T) * (Xe Wu^T), ye = h Wd^T, where Xe holds the
// rows of the expert's tokens. Tiles of 64 tokens x 128 rows of gate and of
// up, or x 256 columns of down; a device-built list of 64-token tiles per
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
// 64-wide k block maps half h, element j to k = 32h + 8s + kSlot[j] (kSlot
// below), so one 16-byte load per lane covers 32 consecutive k of one weight
// row (4 K-steps) and 64 bytes of its activation row, which is stored in
// slot order. Accumulator element j of lane l is
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
// operand slot order kSlot: slot j holds column kSlot[j] = 0 2 4 6 1 3 5 7, so
// each output word is one byte permute of the even or the odd nibbles with
// the constant exponent byte 0x43.
__device__ __forceinline__ bf16x8 nib8_to_bf16(uint32_t w) {
    const uint32_t lo = (w ^ 0x88888888u) & 0x0F0F0F0Fu;          // q + 8 of columns 0, 2, 4, 6
    const uint32_t hi = ((w >> 4) ^ 0x08888888u) & 0x0F0F0F0Fu;   // q + 8 of columns 1, 3, 5, 7
    uint4 r;
    r.x = __builtin_amdgcn_perm(0x43434343u, lo, 0x05010400u);         // 128+u0, 128+u2
    r.y = __builtin_amdgcn_perm(0x43434343u, lo, 0x05030402u);         // 128+u4, 128+u6
    r.z = __builtin_amdgcn_perm(0x43434343u, hi, 0x05010400u);         // 128+u1, 128+u3
    r.w = __builtin_amdgcn_perm(0x43434343u, hi, 0x05030402u);         // 128+u5, 128+u7
    return __builtin_bit_cast(bf16x8, r);
}

// The bf16 activations (x and h) are stored in the same slot order inside
// every aligned group of 8 columns, so an operand is one plain 16-byte load:
// column c lives at position slot_pos(c).
__device__ __forceinline__ int slot_pos(int c) {
    return (c & ~7) + ((c & 7) >> 1) + 4 * (c & 1);
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
// each 64-column group). One thread per 8 columns (two 16-byte loads, lanes
// reading consecutive bytes); the 8 partial sums of a group sit in 8 adjacent
// lanes and are added in a fixed tree order (DPP partners 1, 2, then 7).
__global__ __launch_bounds__(256) void prep_kernel(const float* __restrict__ x, int T, int H,
                                                   uint16_t* __restrict__ xb,
                                                   float* __restrict__ sx) {
    const int C8 = H / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool ok = gid < (int64_t)T * C8;
    const int64_t gc = ok ? gid : (int64_t)T * C8 - 1;
    const int64_t t = gc / C8;
    const int c8 = (int)(gc % C8);
    const float* src = x + t * H + c8 * 8;
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 b = *reinterpret_cast<const float4*>(src + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    // slot order: positions 0..7 hold columns 0 2 4 6 1 3 5 7
    uint32_t pk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c0 = 4 * (i & 1) + (i >> 1), c1 = c0 + 2;     // (0,2) (4,6) (1,3) (5,7)
        pk[i] = (uint32_t)bf16_bits(v[c0]) | ((uint32_t)bf16_bits(v[c1]) << 16);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += bf16_round(v[i]);
    s += __int_as_float(lane_xchg<1>(__float_as_int(s)));
    s += __int_as_float(lane_xchg<2>(__float_as_int(s)));
    s += __int_as_float(lane_xchg<4>(__float_as_int(s)));       // partner lane ^ 7
    if (ok) {
        *reinterpret_cast<uint4*>(xb + t * H + c8 * 8) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        if ((c8 & 7) == 0) sx[t * (H / 64) + c8 / 8] = s;
    }
}

// ------------------------------------------------------------ tile list
// (item, first token) of every 64-token tile, items in order. Items with at
// most gv_max tokens get no tiles: they are compacted, in order, into the
// GEMV work list gv_items / *n_gv (gv_max 0: every item takes tiles).
__global__ __launch_bounds__(256) void tiles_kernel(const WorkItem* __restrict__ items,
                                                    const int32_t* __restrict__ n_items,
                                                    int2* __restrict__ tiles,
                                                    int32_t* __restrict__ n_tiles, int gv_max,
                                                    WorkItem* __restrict__ gv_items,
                                                    int32_t* __restrict__ n_gv) {
    __shared__ int sh[256];
    __shared__ int sg[256];
    const int t = threadIdx.x;
    const int ni = *n_items;
    int base = 0, gbase = 0;
    for (int i0 = 0; i0 < ni; i0 += 256) {
        const int i = i0 + t;
        WorkItem it{};
        if (i < ni) it = items[i];
        const bool small = i < ni && it.count <= gv_max;
        const int c = (i < ni && !small) ? (it.count + kTileM - 1) / kTileM : 0;
        sh[t] = c;
        sg[t] = small ? 1 : 0;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            const int add = t >= o ? sh[t - o] : 0;
            const int addg = t >= o ? sg[t - o] : 0;
            __syncthreads();
            sh[t] += add;
            sg[t] += addg;
            __syncthreads();
        }
        const int start = base + sh[t] - c;
        for (int j = 0; j < c; ++j) tiles[start + j] = make_int2(i, j * kTileM);
        if (small) gv_items[gbase + sg[t] - 1] = it;
        base += sh[255];
        gbase += sg[255];
        __syncthreads();
    }
    if (t == 0) {
        *n_tiles = base;
        *n_gv = gbase;
    }
}

constexpr int kCsChunk = 64;        // 64-column groups staged in LDS at a time (gs64)

// Stage -136 * sums[row(m0 + t)][q] for the 64 tile rows t and the groups
// q = q0 .. q0 + 63 (clamped to n_groups) as s[t * 64 + q - q0]. Called by the
// whole workgroup at the same k block; the barriers fence the previous chunk's
// readers and publish the new one.
__device__ __forceinline__ void stage_group_sums(float* s, const float* sums, const int* rows,
                                                 const WorkItem& it, int m0, int n_groups, int q0) {
    __syncthreads();
    const int nq = min(kCsChunk, n_groups - q0);
    for (int i = threadIdx.x; i < kTileM * kCsChunk; i += blockDim.x) {
        const int t = i / kCsChunk, q = i % kCsChunk;
        if (q < nq) {
            const int r = rows[it.begin + min(m0 + t, it.count - 1)];
            s[i] = -kOffset * sums[(size_t)r * n_groups + q0 + q];
        }
    }
    __syncthreads();
}

// ------------------------------------------------------------ work order
// Work unit = (64-token tile, block of weight rows). Units are taken in a
// grouped order: kGroupTiles consecutive tiles (usually of one expert, or of a
// few small ones) times every row block, so that the units of a group share
// activation rows and weight rows. Workgroup L runs on XCD L % 8; the groups
// are dealt round-robin over the XCDs (XCD x takes groups x, x + 8, ...), so a
// group's reuse stays inside one XCD's L2 and every XCD starts on the first,
// largest experts. Returns false for units past the device-side tile count.
constexpr int kGroupTiles = 2;

__device__ __forceinline__ bool unit_of(int n_tiles, int n_rb, int& tile, int& rb) {
    const int gsz = kGroupTiles * n_rb;                      // units per group
    const int n_groups = (n_tiles + kGroupTiles - 1) / kGroupTiles;
    const int xcd = (int)(blockIdx.x & 7), local = (int)(blockIdx.x >> 3);
    const int grp = (local / gsz) * 8 + xcd;                 // XCD x takes groups x, x + 8, ...
    if (grp >= n_groups) return false;
    const int r = local % gsz;
    const int gt = min(kGroupTiles, n_tiles - grp * kGroupTiles);
    if (r >= gt * n_rb) return false;
    rb = r / gt;
    tile = grp * kGroupTiles + r % gt;
    return true;
}

// ------------------------------------------------------------- main loop
// One wave computes a 64-token x (2 x 32)-row block of sums
//   acc[b][half][j] = sum_k (136 + q_b[n][k]) * A[m][k]
// for its two 32-row weight blocks b (gate and up rows, or two column blocks
// of down) and the tile's token halves (the second only when TWO). The 64 x 64
// activation block of each k step is staged once per workgroup in LDS (double
// buffered, one barrier per k step) and shared by the 4 waves. Weight nibbles
// pass through the wave's own LDS region in whole cache lines (half lines
// with gs64). With GS, every k step is one 64-column scale group, and `out`
// counts in units of the current group's scale: at each group the sums so far
// are rescaled by (previous scale / this scale) and take the group's -136 * S
// correction (read from LDS), and at the end they are multiplied by the last
// scale; otherwise `out` holds the raw sums.
constexpr int kLdsRow = 72;          // bf16 per LDS activation row (64 + 8 pad: conflict-free 16-B reads)
constexpr int kSB = 4 * 2 * 32 * 128;  // bytes of the per-wave weight-line regions of a workgroup

// Lane `src`'s pointer (a 64-bit value through two 32-bit shuffles).
__device__ __forceinline__ const uint8_t* shfl_ptr(const uint8_t* p, int src) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src);
    const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src);
    return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}

template <bool GS, bool TWO, int GL>
__device__ __forceinline__ void mainloop(const uint16_t* __restrict__ arow, int nk,
                                         const uint8_t* __restrict__ b0, const uint8_t* __restrict__ b1,
                                         const float* __restrict__ gs0, const float* __restrict__ gs1,
                                         const float* __restrict__ sums, const int32_t* __restrict__ rows,
                                         const WorkItem& it, int m0,
                                         uint16_t (*sA)[kTileM][kLdsRow], float* s_cs,
                                         uint8_t* sB, f32x16 (&out)[2][2]) {
    const int lane = threadIdx.x & 63, ln = lane & 31, lh = lane >> 5;
    const int ar = threadIdx.x >> 2, aq = threadIdx.x & 3;     // staging: row, 16-column quarter
    const bool aload = TWO || ar < 32;                         // wave-uniform
    // the sums accumulate straight into `out`: with per-row scales as raw sums,
    // with gs64 in units of the current group's scale (rescaled at each group)
    f32x16 (&acc)[2][2] = out;
#pragma unroll
    for (int b = 0; b < 2; ++b) out[b][0] = out[b][1] = f32x16{};
    // activation rows run kA k steps ahead (2; 1 with gs64 half lines, for
    // registers): register set k % kA holds k step k between its load and its
    // store to LDS at the end of step k - 1
    constexpr int kA = (GS && GL == 2) ? 1 : 2;
    // gs64: the group scales of the weight rows run kF k steps ahead
    constexpr int kF = 2;
    uint4 Ar[kA][2] = {};
    float F[kF][2] = {};                                       // gs64: scales of the staged k steps
    auto ldA = [&](int set, int kb) {
        if (aload) {
            Ar[set][0] = ldg16(arow + kb * 64);
            Ar[set][1] = ldg16(arow + kb * 64 + 8);
        }
    };
    auto stA = [&](int buf, int set) {
        if (aload) {
            *reinterpret_cast<uint4*>(&sA[buf][ar][aq * 16]) = Ar[set][0];
            *reinterpret_cast<uint4*>(&sA[buf][ar][aq * 16 + 8]) = Ar[set][1];
        }
    };
    auto ldF = [&](float (&F)[2], int kb) {
        F[0] = gs0[kb];
        F[1] = gs1[kb];
    };
    auto mma = [&](int buf, const uint4 (&P)[2]) {
        const uint4* r0 = reinterpret_cast<const uint4*>(&sA[buf][ln][lh * 32]);
        const uint4* r1 = reinterpret_cast<const uint4*>(&sA[buf][32 + ln][lh * 32]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint4 a0 = r0[s];
            uint4 a1;
            if (TWO) a1 = r1[s];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const uint32_t w = s == 0 ? P[b].x : s == 1 ? P[b].y : s == 2 ? P[b].z : P[b].w;
                const bf16x8 bb = nib8_to_bf16(w);
                acc[b][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), bb, acc[b][0], 0, 0, 0);
                if (TWO) acc[b][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1), bb, acc[b][1], 0, 0, 0);
            }
        }
    };
    // gs64: the group of k step kb starts from the sums so far in units of its
    // own scale, acc * (previous scale / this scale), plus its -136 * S
    // correction (staged in LDS); an all-zero group (scale 0) keeps the
    // previous unit. Then out = sum_g scale_g * P_g = acc * (last scale).
    float unit[2] = {0.f, 0.f};                                // the scale acc is counted in, per row
    auto regroup = [&](int kb, const float (&f)[2]) {
        const float* cs_k = s_cs + kb % kCsChunk;
        float ratio[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const float fe = f[b] != 0.f ? f[b] : unit[b];
            ratio[b] = (kb == 0 || fe == 0.f) ? 0.f : unit[b] * __builtin_amdgcn_rcpf(fe);
            unit[b] = fe;
        }
#pragma unroll
        for (int mb = 0; mb < (TWO ? 2 : 1); ++mb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float cs = cs_k[(mb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3)) * kCsChunk];
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[b][mb][j] = fmaf(acc[b][mb][j], ratio[b], cs);
            }
    };
    const int last = nk - 1;
    ldA(0, 0);
#pragma unroll
    for (int j = 1; j < kA; ++j) ldA(j, min(j, last));
    stA(0, 0);
    if constexpr (GS) {
#pragma unroll
        for (int j = 0; j < kF; ++j) ldF(F[j], min(j, last));
    }
    // Weight rows go through the wave's own LDS region in whole (GL = 4) or
    // half (GL = 2) cache lines. Every GL k steps the wave requests the next
    // GL steps of its 64 rows (gate and up, or two column blocks of down): a
    // load of RPI rows
    // x GL * 32 bytes touches RPI lines and uses GL * 32 bytes of each, where
    // the MFMA operand layout would touch 32 lines and use 32 bytes of each.
    // At the end of a group the wave stores the next group into its region
    // (16-byte chunks XOR-swizzled by row, so that eight consecutive rows fall
    // on distinct banks for the operand reads below) and each k step reads its
    // operands from there. Only the wave itself reads its region, and one
    // wave's LDS operations execute in order, so no barrier is needed.
    static_assert(GL == 2 || GL == 4, "k steps per load group");
    constexpr int NG = 2 * GL;                                 // 16-byte chunks per row and group
    constexpr int RPI = 64 / NG;                               // rows per load
    constexpr int NI = 32 / RPI;                               // loads per matrix and group
    auto swz = [](int r) { return (r / (16 / NG)) & (NG - 1); };
    uint8_t* sBw = sB + (threadIdx.x >> 6) * (2 * 32 * 16 * NG);
    const int rowbytes = nk * 32;                              // bytes of one weight row
    // rows q * RPI + lane / NG as byte offsets from the wave's first row
    // (each taken from a lane of that row with lh == 0)
    const uint8_t* base[2] = {shfl_ptr(b0, 0), shfl_ptr(b1, 0)};
    uint32_t ro[2][NI];
#pragma unroll
    for (int q = 0; q < NI; ++q) {
        const int src = q * RPI + lane / NG;
        ro[0][q] = (uint32_t)(shfl_ptr(b0, src) - base[0]);
        ro[1][q] = (uint32_t)(shfl_ptr(b1, src) - base[1]);
    }
    uint4 Q[2][NI];
    auto ldG = [&](int g) {
        const uint32_t off = (uint32_t)min(g * GL * 32 + (lane % NG) * 16, rowbytes - 16);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int q = 0; q < NI; ++q) Q[m][q] = ldg16(base[m] + (ro[m][q] + off));
    };
    auto stG = [&]() {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int q = 0; q < NI; ++q) {
                const int r = q * RPI + lane / NG;
                *reinterpret_cast<uint4*>(sBw + (m * 32 + r) * (16 * NG) + (((lane % NG) ^ swz(r)) * 16)) = Q[m][q];
            }
    };
    auto ldP = [&](int d, uint4 (&Pk)[2]) {                    // k step d of the group: its 32 bytes
        const int c = d * 2 + lh;
#pragma unroll
        for (int m = 0; m < 2; ++m)
            Pk[m] = *reinterpret_cast<const uint4*>(sBw + (m * 32 + ln) * (16 * NG) + ((c ^ swz(ln)) * 16));
    };
    const int ng = (nk + GL - 1) / GL, last_g = ng - 1;
    // one k step (k & 1 == d & 1 == the LDS activation buffer): request the
    // activation block kA steps ahead, multiply the current one with the
    // step's weights (gs64: after rescaling the sums to the step's group and
    // requesting the scales kF steps ahead); store the next activation block
    auto kstep = [&](int k, int d, bool group_end, int g) {
        if (GS && k % kCsChunk == 0) stage_group_sums(s_cs, sums, rows, it, m0, nk, k);
        ldA(k % kA, min(k + kA, last));
        if (kA >= 2) asm volatile("" ::: "memory");
        if constexpr (GS) {
            regroup(k, F[d % kF]);
            ldF(F[d % kF], min(k + kF, last));
        }
        uint4 Pk[2];
        ldP(d, Pk);
        // gs64 (VALU regrouping between the MFMA blocks): the wave with MFMAs
        // to issue goes first (measured 2% faster; with per-row scales it
        // measured slower)
        if constexpr (GS) __builtin_amdgcn_s_setprio(1);
        mma(d & 1, Pk);
        if constexpr (GS) __builtin_amdgcn_s_setprio(0);
        stA((d & 1) ^ 1, (k + 1) % kA);
        if (group_end) {
            stG();
            ldG(min(g + 2, last_g));
        }
        __syncthreads();
    };
    ldG(0);
    stG();
    ldG(min(1, last_g));
    __syncthreads();
    int g = 0;
    for (; g < last_g; ++g) {
#pragma unroll
        for (int d = 0; d < GL; ++d) kstep(g * GL + d, d, d == GL - 1, g);
    }
#pragma unroll
    for (int d = 0; d < GL; ++d)
        if (g * GL + d < nk) kstep(g * GL + d, d, false, g);
    if constexpr (GS) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int mb = 0; mb < (TWO ? 2 : 1); ++mb)
#pragma unroll
                for (int j = 0; j < 16; ++j) out[b][mb][j] *= unit[b];
    }
}

// ----------------------------------------------------------------- gate/up
// Workgroup: 64 tokens of one item x 128 intermediate rows of gate and up.
// Wave w owns rows 32w..32w+31 of both matrices; epilogue h = silu(g) * u,
// stored as bf16 by output row, plus the per-64-row sums of the stored bf16
// values that the down GEMM's correction needs.
template <bool GS, bool TWO>
__device__ __forceinline__ void gateup_tile(const GemmArgs& a, const WorkItem& it, int m0, int rb,
                                            uint16_t (*sA)[kTileM][kLdsRow], float* s_cs, uint8_t* sB,
                                            const float* s_tot, const int* s_out,
                                            float (*s_part)[kTileM]) {
    const int H = a.H, I = a.I, G = H / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ln = lane & 31, lh = lane >> 5;
    const BlobLayout& L = a.L;
    const int wrow = rb * 128 + wave * 32;                    // this wave's first weight row
    const bool wlive = wrow < I;                              // false in the last block when I % 128 == 64
    const int irow = min(wrow, I - 32) + ln;                  // this lane's weight row (clamped when dead)
    const size_t boff = (size_t)gu_row(irow) * (H / 2) + lh * 16;
    const float* gsc = reinterpret_cast<const float*>(it.blob + L.gate_s);
    const float* usc = reinterpret_cast<const float*>(it.blob + L.up_s);
    const int atok = a.rows_tok[it.begin + min(m0 + (int)(threadIdx.x >> 2), it.count - 1)];
    const uint16_t* arow = a.xb + (size_t)atok * H + (threadIdx.x & 3) * 16;

    // per-row scales are read before the main loop: in the epilogue a late
    // load would make every store wait for the stores before it
    const float fg = GS ? 1.f : gsc[irow], fu = GS ? 1.f : usc[irow];
    f32x16 out[2][2];
    mainloop<GS, TWO, 4>(arow, G, it.blob + L.gate_q + boff, it.blob + L.up_q + boff,
                      gsc + (size_t)irow * G, usc + (size_t)irow * G, a.sx, a.rows_tok, it, m0,
                      sA, s_cs, sB, out);

#pragma unroll
    for (int mb = 0; mb < (TWO ? 2 : 1); ++mb) {
        float rsum[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int mi = mb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);     // token in the tile
            const float g = GS ? out[0][mb][j] : fg * (out[0][mb][j] - kOffset * s_tot[mi]);
            const float u = GS ? out[1][mb][j] : fu * (out[1][mb][j] - kOffset * s_tot[mi]);
            const float h = g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
            rsum[j] = bf16_round(h);
            const int o = s_out[mi];
            if (o >= 0 && wlive) a.hb[(size_t)o * I + slot_pos(irow)] = bf16_bits(h);
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
            for (int j = 0; j < 16; ++j) s_part[wave][mb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3)] = rsum[j];
        }
    }
    __syncthreads();
    // group sums: waves (0, 1) cover one 64-row group of h, waves (2, 3) the next
    if (threadIdx.x < 2 * kTileM) {
        const int t = threadIdx.x & (kTileM - 1), grp = threadIdx.x >> 6;
        const int o = s_out[t], q = rb * 2 + grp;
        if (o >= 0 && q * 64 < I) a.sh[(size_t)o * (I / 64) + q] = s_part[2 * grp][t] + s_part[2 * grp + 1][t];
    }
}

// Three resident waves per SIMD with per-row scales (three workgroups per CU
// also fit the LDS), two with gs64: its whole-line weight staging needs more
// registers than three allow, and half lines (three waves) were fetched twice
// from memory, the line evicted between its two halves (11.2 GB of L2 misses
// per call against 5.6), which cost more than the lower occupancy.
template <bool GS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(GS ? 2 : 3)))
void gemm_gateup_kernel(GemmArgs a) {
    __shared__ __align__(16) uint16_t sA[2][kTileM][kLdsRow];
    __shared__ __align__(16) uint8_t sB[kSB];    // the waves' weight-line regions
    __shared__ float s_part[4][kTileM];          // per-wave token sums of bf16(h)
    __shared__ float s_tot[kTileM];              // per-token sum of the bf16 x row
    __shared__ int s_out[kTileM];                // output row of each tile row, -1 past the item
    __shared__ float s_cs[GS ? kTileM * kCsChunk : 1];   // gs64: -136 * group sums, [token][group]
    int tile, rb;
    if (!unit_of(*a.n_tiles, (a.I + 127) / 128, tile, rb)) return;
    const int2 td = a.tiles[tile];
    const WorkItem it = a.items[td.x];
    const int m0 = td.y;
    if (threadIdx.x < kTileM) {
        const int m = m0 + (int)threadIdx.x;
        s_out[threadIdx.x] = m < it.count ? a.rows_out[it.begin + m] : -1;
    }
    if (!GS && threadIdx.x < kTileM) {
        const int G = a.H / 64;
        const int tok = a.rows_tok[it.begin + min(m0 + (int)threadIdx.x, it.count - 1)];
        float s = 0.f;
        for (int q = 0; q < G; ++q) s += a.sx[(size_t)tok * G + q];
        s_tot[threadIdx.x] = s;
    }
    // (the main loop's first barrier publishes s_tot)
    if (it.count - m0 > 32) gateup_tile<GS, true>(a, it, m0, rb, sA, s_cs, sB, s_tot, s_out, s_part);
    else gateup_tile<GS, false>(a, it, m0, rb, sA, s_cs, sB, s_tot, s_out, s_part);
}

// -------------------------------------------------------------------- down
// Workgroup: 64 tokens of one item x 256 output columns. Wave w owns columns
// 64w..64w+63 as two 32-column blocks.
template <bool GS, bool TWO>
__device__ __forceinline__ void down_tile(const GemmArgs& a, const WorkItem& it, int m0, int rb,
                                          uint16_t (*sA)[kTileM][kLdsRow], float* s_cs, uint8_t* sB,
                                          const float* s_tot, const int* s_out) {
    const int H = a.H, I = a.I, GI = I / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ln = lane & 31, lh = lane >> 5;
    const BlobLayout& L = a.L;
    const uint8_t* dq = it.blob + L.down_q;
    const float* dsc = reinterpret_cast<const float*>(it.blob + L.down_s);
    const int c0 = rb * 256 + wave * 64 + ln, c1 = c0 + 32;   // this lane's two output columns
    const int cc0 = min(c0, H - 1), cc1 = min(c1, H - 1);
    const int arw = a.rows_out[it.begin + min(m0 + (int)(threadIdx.x >> 2), it.count - 1)];
    const uint16_t* arow = a.hb + (size_t)arw * I + (threadIdx.x & 3) * 16;

    const float f[2] = {GS ? 1.f : dsc[cc0], GS ? 1.f : dsc[cc1]};   // before the loop, as in gate/up
    f32x16 out[2][2];
    mainloop<GS, TWO, GS ? 2 : 4>(arow, GI, dq + (size_t)cc0 * (I / 2) + lh * 16, dq + (size_t)cc1 * (I / 2) + lh * 16,
                      dsc + (size_t)cc0 * GI, dsc + (size_t)cc1 * GI, a.sh, a.rows_out, it, m0,
                      sA, s_cs, sB, out);

    const int cols[2] = {c0, c1};
#pragma unroll
    for (int mb = 0; mb < (TWO ? 2 : 1); ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int mi = mb * 32 + 8 * (j >> 2) + 4 * lh + (j & 3);
            const int o = s_out[mi];
            if (o < 0) continue;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                if (cols[b] >= H) continue;
                const float y = GS ? out[b][mb][j] : f[b] * (out[b][mb][j] - kOffset * s_tot[mi]);
                a.y_rows[(size_t)o * H + cols[b]] = y;
            }
        }
}

// Three resident waves per SIMD; with gs64 the weights go in half lines (the
// whole-line staging's registers would leave two waves, which measured slower
// here than the lines fetched twice).
template <bool GS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void gemm_down_kernel(GemmArgs a) {
    __shared__ __align__(16) uint16_t sA[2][kTileM][kLdsRow];
    __shared__ __align__(16) uint8_t sB[GS ? kSB / 2 : kSB];    // the waves' weight-line regions (half lines with gs64)
    __shared__ float s_tot[kTileM];              // per-row sum of the bf16 h row
    __shared__ int s_out[kTileM];                // output row of each tile row, -1 past the item
    __shared__ float s_cs[GS ? kTileM * kCsChunk : 1];   // gs64: -136 * group sums, [row][group]
    int tile, rb;
    if (!unit_of(*a.n_tiles, (a.H + 255) / 256, tile, rb)) return;
    const int2 td = a.tiles[tile];
    const WorkItem it = a.items[td.x];
    const int m0 = td.y;
    if (threadIdx.x < kTileM) {
        const int m = m0 + (int)threadIdx.x;
        s_out[threadIdx.x] = m < it.count ? a.rows_out[it.begin + m] : -1;
    }
    if (!GS && threadIdx.x < kTileM) {
        const int GI = a.I / 64;
        const int o = a.rows_out[it.begin + min(m0 + (int)threadIdx.x, it.count - 1)];
        float s = 0.f;
        for (int q = 0; q < GI; ++q) s += a.sh[(size_t)o * GI + q];
        s_tot[threadIdx.x] = s;
    }
    if (it.count - m0 > 32) down_tile<GS, true>(a, it, m0, rb, sA, s_cs, sB, s_tot, s_out);
    else down_tile<GS, false>(a, it, m0, rb, sA, s_cs, sB, s_tot, s_out);
}

}  // namespace

// Workgroups per XCD for unit_of: whole groups, the groups dealt round-robin.
static size_t unit_slots(int32_t max_tiles, int n_rb) {
    const size_t n_groups = ((size_t)max_tiles + kGroupTiles - 1) / kGroupTiles;
    return (n_groups + 7) / 8 * (size_t)kGroupTiles * (size_t)n_rb;
}

size_t gemm_tiles_max(int32_t rows, int32_t max_items) {
    return (size_t)rows / kTileM + (size_t)max_items + 1;
}

coli_status launch_mfma_ffn(const GemmArgs& a, const float* x, int32_t T, int32_t max_tiles,
                            hipStream_t stream) {
    if (a.H % 64 || a.I % 64) return fail(COLI_EUNSUPPORTED, "mfma path: hidden and inter must be multiples of 64");
    const int64_t prep_threads = (int64_t)T * (a.H / 8);
    launch(prep_kernel, dim3((unsigned)((prep_threads + 255) / 256)), dim3(256), 0, stream, x, T,
           a.H, a.xb, a.sx);
    COLI_CHECK_LAUNCH("prep kernel launch");
    launch(tiles_kernel, dim3(1), dim3(256), 0, stream, a.items, a.n_items, a.tiles, a.n_tiles,
           a.gv_max, a.gv_items, a.n_gv);
    COLI_CHECK_LAUNCH("tile list kernel launch");
    {
        ProfTag prof("gemm_gateup");
        const dim3 grid((unsigned)(8 * unit_slots(max_tiles, (a.I + 127) / 128)));
        if (a.group) launch(gemm_gateup_kernel<true>, grid, dim3(256), 0, stream, a);
        else launch(gemm_gateup_kernel<false>, grid, dim3(256), 0, stream, a);
    }
    COLI_CHECK_LAUNCH("gate/up GEMM launch");
    {
        ProfTag prof("gemm_down");
        const dim3 grid((unsigned)(8 * unit_slots(max_tiles, (a.H + 255) / 256)));
        if (a.group) launch(gemm_down_kernel<true>, grid, dim3(256), 0, stream, a);
        else launch(gemm_down_kernel<false>, grid, dim3(256), 0, stream, a);
    }
    COLI_CHECK_LAUNCH("down GEMM launch");
    return COLI_OK;
}

}  // namespace coli
