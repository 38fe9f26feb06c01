// Batch union (lbrq.cn article section 三 item 4; practical guide section 二):
// the T*k (token, slot) assignments are grouped by expert so that each
// unique expert's weights are read once for all of its tokens.
//
// Three passes over slabs of 1024 assignments, deterministic throughout:
//  1. per slab (one workgroup, 16 waves of 64): lanes holding the same expert
//     are found with ballots (one round per distinct expert in the wave),
//     which gives each assignment its rank among equal experts of its wave and
//     the wave's per-expert count; an exclusive scan over the 16 waves (in
//     order) turns that into the rank inside the slab and the slab's count;
//  2. one workgroup: per expert, an exclusive scan of the slab counts (in slab
//     order), the expert's total, then offsets (exclusive scan over experts)
//     and the unique list;
//  3. per slab: perm[offsets[e] + slab_prefix[s][e] + rank] = a.
// The result is the stable counting sort of the assignments by expert.
#include <algorithm>

#include "common.h"

namespace coli {
namespace {

constexpr int kUnionThreads = 1024;
constexpr int kSlab = kUnionThreads;           // assignments per slab
constexpr int kSlabWaves = kSlab / 64;

__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int* total) {
    // Hillis-Steele over 1024 threads; sh has 1024 ints.
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (int o = 1; o < kUnionThreads; o <<= 1) {
        int add = (t >= o) ? sh[t - o] : 0;
        __syncthreads();
        sh[t] += add;
        __syncthreads();
    }
    const int incl = sh[t];
    *total = sh[kUnionThreads - 1];
    __syncthreads();
    return incl - v;
}

__device__ __forceinline__ int valid_expert(const int32_t* idx, int a, int n, int E) {
    const int e = a < n ? idx[a] : -1;
    return (e >= 0 && e < E) ? e : -1;           // out-of-range entries are skipped
}

// Pass 1. Dynamic LDS: kSlabWaves * E ints.
__global__ __launch_bounds__(kUnionThreads) void union_count_kernel(
    const int32_t* __restrict__ idx, int n, int E, int32_t* __restrict__ slab_cnt /* [S][E] */,
    int32_t* __restrict__ rank /* [n] */) {
    extern __shared__ int s_cnt[];               // [wave][E]: counts, then exclusive prefixes
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    for (int i = t; i < kSlabWaves * E; i += kUnionThreads) s_cnt[i] = 0;
    __syncthreads();
    const int a = blockIdx.x * kSlab + t;
    const int e = valid_expert(idx, a, n, E);
    int r = 0;
    unsigned long long active = __ballot(e >= 0);
    while (active) {
        const int leader = __ffsll((long long)active) - 1;
        const int v = __shfl(e, leader);
        const unsigned long long m = __ballot(e == v) & active;
        if (e == v) r = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == leader) s_cnt[wave * E + v] = __popcll(m);
        active &= ~m;
    }
    __syncthreads();
    for (int x = t; x < E; x += kUnionThreads) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kSlabWaves; ++w) {
            const int v = s_cnt[w * E + x];
            s_cnt[w * E + x] = c;
            c += v;
        }
        slab_cnt[(int64_t)blockIdx.x * E + x] = c;
    }
    __syncthreads();
    if (e >= 0) rank[a] = s_cnt[wave * E + e] + r;
}

// Pass 2: one workgroup.
__global__ __launch_bounds__(kUnionThreads) void union_scan_kernel(
    int S, int E, int32_t* __restrict__ slab_cnt, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ unique, int32_t* __restrict__ n_unique) {
    __shared__ int sh[kUnionThreads];
    const int t = threadIdx.x;
    int cnt = 0;
    if (t < E) {
        int s = 0;
        for (; s + 8 <= S; s += 8) {             // independent loads, then the serial sum
            int v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = slab_cnt[(int64_t)(s + j) * E + t];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                slab_cnt[(int64_t)(s + j) * E + t] = cnt;
                cnt += v[j];
            }
        }
        for (; s < S; ++s) {
            const int v = slab_cnt[(int64_t)s * E + t];
            slab_cnt[(int64_t)s * E + t] = cnt;
            cnt += v;
        }
        counts[t] = cnt;
    }
    int total = 0;
    const int off = block_exclusive_scan(t < E ? cnt : 0, sh, &total);
    if (t < E) offsets[t] = off;
    if (t == 0) offsets[E] = total;
    int nu = 0;
    const int upos = block_exclusive_scan((t < E && cnt > 0) ? 1 : 0, sh, &nu);
    if (t < E && cnt > 0) unique[upos] = t;
    if (t == 0) *n_unique = nu;
}

// Pass 3.
__global__ __launch_bounds__(kUnionThreads) void union_scatter_kernel(
    const int32_t* __restrict__ idx, int n, int E, const int32_t* __restrict__ slab_cnt,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm) {
    const int a = blockIdx.x * kSlab + threadIdx.x;
    const int e = valid_expert(idx, a, n, E);
    if (e < 0) return;
    perm[offsets[e] + slab_cnt[(int64_t)blockIdx.x * E + e] + rank[a]] = a;
}

// Work list for the FFN kernels: optional shared expert first, then the
// unique experts in ascending order (optionally only those of one phase).
// Every workgroup fills 256 rows of the slot list; workgroup 0 builds the list.
__global__ __launch_bounds__(256) void plan_kernel(
    const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ unique,
    const int32_t* __restrict__ n_unique, const void* const* __restrict__ table,
    const void* shared_blob, int T, int k, const uint8_t* __restrict__ phase_mask,
    int phase, WorkItem* __restrict__ items, int32_t* __restrict__ n_items,
    int32_t* __restrict__ rows_tok, int32_t* __restrict__ rows_out) {
    __shared__ int sh[256];
    const int t = threadIdx.x;
    const int n = T * k;
    const int p = blockIdx.x * 256 + t;          // slot-list rows: one per thread over the grid
    if (p < n) {
        const int a = perm[p];
        rows_tok[p] = a / k;
        rows_out[p] = a;
    } else if (p < n + T) {
        rows_tok[p] = p - n;
        rows_out[p] = p;
    }
    if (blockIdx.x != 0) return;
    const int has_shared = shared_blob != nullptr ? 1 : 0;
    if (t == 0 && has_shared) {
        WorkItem it;
        it.blob = (const uint8_t*)shared_blob;
        it.begin = n;
        it.count = T;
        it.row0 = n;
        items[0] = it;
    }
    // compaction of the unique list by phase, in order, 256 at a time
    const int nu = *n_unique;
    int base = has_shared;
    for (int u0 = 0; u0 < nu; u0 += 256) {
        const int u = u0 + t;
        int keep = 0, e = 0;
        if (u < nu) {
            e = unique[u];
            keep = (phase_mask == nullptr || phase_mask[e] == phase) ? 1 : 0;
        }
        sh[t] = keep;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            int add = (t >= o) ? sh[t - o] : 0;
            __syncthreads();
            sh[t] += add;
            __syncthreads();
        }
        const int pos = sh[t] - keep;
        const int tot = sh[255];
        if (keep) {
            WorkItem it;
            it.blob = (const uint8_t*)table[e];
            it.begin = offsets[e];
            it.count = offsets[e + 1] - offsets[e];
            it.row0 = perm[offsets[e]];
            items[base + pos] = it;
        }
        base += tot;
        __syncthreads();
    }
    if (t == 0) *n_items = base;
}

}  // namespace

size_t union_ws_bytes(int32_t T, int32_t k, int32_t E) {
    const size_t n = (size_t)T * k, S = (n + kSlab - 1) / kSlab;
    return align256(S * (size_t)E * 4) + align256(n * 4 + 4);
}

coli_status launch_union(const int32_t* idx, int32_t T, int32_t k, int32_t E, int32_t* counts,
                         int32_t* offsets, int32_t* perm, int32_t* unique, int32_t* n_unique,
                         void* ws, hipStream_t stream) {
    const int n = T * k;
    const int S = (n + kSlab - 1) / kSlab;
    int32_t* slab_cnt = (int32_t*)ws;
    int32_t* rank = (int32_t*)((char*)ws + align256((size_t)S * E * 4));
    if (S > 0) {
        launch(union_count_kernel, dim3(S), dim3(kUnionThreads), (size_t)kSlabWaves * E * 4, stream,
               idx, n, E, slab_cnt, rank);
        COLI_CHECK_LAUNCH("union count kernel launch");
    }
    launch(union_scan_kernel, dim3(1), dim3(kUnionThreads), 0, stream, S, E, slab_cnt, counts,
           offsets, unique, n_unique);
    COLI_CHECK_LAUNCH("union scan kernel launch");
    if (S > 0) {
        launch(union_scatter_kernel, dim3(S), dim3(kUnionThreads), 0, stream, idx, n, E, slab_cnt,
               rank, offsets, perm);
        COLI_CHECK_LAUNCH("union scatter kernel launch");
    }
    return COLI_OK;
}

coli_status launch_plan(const int32_t* offsets, const int32_t* perm,
                        const int32_t* unique, const int32_t* n_unique,
                        const void* const* blob_table, const void* shared_blob, int32_t T,
                        int32_t k, int32_t E, const uint8_t* phase_mask, int32_t phase,
                        WorkItem* items, int32_t* n_items, int32_t* rows_tok, int32_t* rows_out,
                        hipStream_t stream) {
    const int rows = T * k + T;
    launch(plan_kernel, dim3(std::max(1, (rows + 255) / 256)), dim3(256), 0, stream, offsets, perm, unique,
                       n_unique, blob_table, shared_blob, T, k, phase_mask, phase, items,
                       n_items, rows_tok, rows_out);
    COLI_CHECK_LAUNCH("plan kernel launch");
    return COLI_OK;
}

}  // namespace coli
