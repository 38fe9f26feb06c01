// Batch union (lbrq.cn article section 三 item 4; practical guide section 二):
// the T*k (token, slot) assignments are grouped by expert so that each
// unique expert's weights are read once for all of its tokens.
//
// One workgroup of 1024 threads, deterministic throughout:
//  1. every wave takes 64-assignment chunks; inside a chunk, lanes holding the
//     same expert are found with ballots (one round per distinct expert), which
//     gives each assignment its rank among equal experts of its chunk and the
//     chunk's per-expert count;
//  2. per expert, an exclusive scan over the chunks (in chunk order);
//  3. counts -> offsets (exclusive scan over experts) and the unique list;
//  4. scatter: perm[offsets[e] + chunk_prefix[c][e] + rank] = a.
// The result is the stable counting sort of the assignments by expert.
#include "common.h"

namespace coli {
namespace {

constexpr int kUnionThreads = 1024;

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

__global__ __launch_bounds__(kUnionThreads) void union_kernel(
    const int32_t* __restrict__ idx, int n, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ unique,
    int32_t* __restrict__ n_unique, int32_t* __restrict__ chunk_cnt /* [C][E] */,
    int32_t* __restrict__ rank /* [n] */) {
    __shared__ int sh[kUnionThreads];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, nwaves = kUnionThreads / 64;
    const int C = (n + 63) / 64;
    for (int i = t; i < C * E; i += kUnionThreads) chunk_cnt[i] = 0;
    __syncthreads();
    // 1. ranks inside each chunk
    for (int c = wave; c < C; c += nwaves) {
        const int a = c * 64 + lane;
        int e = (a < n) ? idx[a] : -1;
        if (e >= E) e = -1;                       // out-of-range entries are skipped
        unsigned long long active = __ballot(e >= 0);
        while (active) {
            const int leader = __ffsll((long long)active) - 1;
            const int v = __shfl(e, leader);
            const unsigned long long m = __ballot(e == v) & active;
            if (e == v) {
                const unsigned long long below = (lane == 0) ? 0ull : (m & ((1ull << lane) - 1ull));
                rank[a] = __popcll(below);
            }
            if (lane == leader) chunk_cnt[(int64_t)c * E + v] = __popcll(m);
            active &= ~m;
        }
    }
    __syncthreads();
    // 2. per-expert exclusive scan over chunks, in chunk order
    int cnt = 0;
    if (t < E) {
        for (int c = 0; c < C; ++c) {
            const int v = chunk_cnt[(int64_t)c * E + t];
            chunk_cnt[(int64_t)c * E + t] = cnt;
            cnt += v;
        }
        counts[t] = cnt;
    }
    __syncthreads();
    // 3. offsets and the unique list
    int total = 0;
    const int off = block_exclusive_scan(t < E ? cnt : 0, sh, &total);
    if (t < E) offsets[t] = off;
    if (t == 0) offsets[E] = total;
    int nu = 0;
    const int upos = block_exclusive_scan((t < E && cnt > 0) ? 1 : 0, sh, &nu);
    if (t < E && cnt > 0) unique[upos] = t;
    if (t == 0) *n_unique = nu;
    // offsets[] of other threads are needed below: keep them in shared memory
    __syncthreads();
    sh[t] = off;
    __syncthreads();
    // 4. scatter
    for (int a = t; a < n; a += kUnionThreads) {
        const int e = idx[a];
        if (e < 0 || e >= E) continue;
        const int c = a / 64;
        perm[sh[e] + chunk_cnt[(int64_t)c * E + e] + rank[a]] = a;
    }
}

// Work list for the FFN kernels: optional shared expert first, then the
// unique experts in ascending order (optionally only those of one phase).
__global__ __launch_bounds__(256) void plan_kernel(
    const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ unique,
    const int32_t* __restrict__ n_unique, const void* const* __restrict__ table,
    const void* shared_blob, int T, int k, int E, const uint8_t* __restrict__ phase_mask,
    int phase, WorkItem* __restrict__ items, int32_t* __restrict__ n_items,
    int32_t* __restrict__ rows_tok, int32_t* __restrict__ rows_out) {
    __shared__ int sh[256];
    const int t = threadIdx.x;
    const int n = T * k;
    for (int p = t; p < n; p += 256) {
        const int a = perm[p];
        rows_tok[p] = a / k;
        rows_out[p] = a;
    }
    for (int s = t; s < T; s += 256) {
        rows_tok[n + s] = s;
        rows_out[n + s] = n + s;
    }
    const int has_shared = shared_blob != nullptr ? 1 : 0;
    if (t == 0 && has_shared) {
        WorkItem it;
        it.blob = (const uint8_t*)shared_blob;
        it.begin = n;
        it.count = T;
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
            items[base + pos] = it;
        }
        base += tot;
        __syncthreads();
    }
    if (t == 0) *n_items = base;
}

}  // namespace

size_t union_ws_bytes(int32_t T, int32_t k, int32_t E) {
    const size_t n = (size_t)T * k, C = (n + 63) / 64;
    return align256(C * (size_t)E * 4) + align256(n * 4 + 4);
}

coli_status launch_union(const int32_t* idx, int32_t T, int32_t k, int32_t E, int32_t* counts,
                         int32_t* offsets, int32_t* perm, int32_t* unique, int32_t* n_unique,
                         void* ws, hipStream_t stream) {
    const int n = T * k;
    const size_t C = ((size_t)n + 63) / 64;
    int32_t* chunk_cnt = (int32_t*)ws;
    int32_t* rank = (int32_t*)((char*)ws + align256(C * (size_t)E * 4));
    launch(union_kernel, dim3(1), dim3(kUnionThreads), 0, stream, idx, n, E, counts,
                       offsets, perm, unique, n_unique, chunk_cnt, rank);
    COLI_CHECK_LAUNCH("union kernel launch");
    return COLI_OK;
}

coli_status launch_plan(const int32_t* offsets, const int32_t* perm,
                        const int32_t* unique, const int32_t* n_unique,
                        const void* const* blob_table, const void* shared_blob, int32_t T,
                        int32_t k, int32_t E, const uint8_t* phase_mask, int32_t phase,
                        WorkItem* items, int32_t* n_items, int32_t* rows_tok, int32_t* rows_out,
                        hipStream_t stream) {
    launch(plan_kernel, dim3(1), dim3(256), 0, stream, offsets, perm, unique,
                       n_unique, blob_table, shared_blob, T, k, E, phase_mask, phase, items,
                       n_items, rows_tok, rows_out);
    COLI_CHECK_LAUNCH("plan kernel launch");
    return COLI_OK;
}

}  // namespace coli
