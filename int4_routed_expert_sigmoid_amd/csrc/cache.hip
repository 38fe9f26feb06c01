// HBM expert cache: a per-layer LRU of expert blobs in a device arena, filled
// from pinned host memory (practical guide section 二: per-layer LRU cache;
// each expert's three matrices are adjacent so a miss is one read; missing
// experts load while resident ones compute; a read in flight is never issued
// twice; placement changes speed only, never routing or results), with the
// learned parts of the same guide's tuning section (section 五): a usage
// history per (layer, expert), pinned experts that share the layer's slots
// with the LRU, pinning of the historically hottest experts, a repin step that
// swaps cold pinned experts for hot ones under hysteresis and a swap limit, and
// prefetch of the experts a router lookahead predicts (PILOT, section 二).
//
// Host-side bookkeeping plus HIP copies and events:
//  - a copy takes the first empty slot, else the least recently used slot that
//    is not pinned and not otherwise excluded (equal ages: the lowest expert
//    id), makes the copy stream wait for the compute that last read that slot
//    (its release event), enqueues one host-to-device copy of the whole blob
//    and the slot's ready event, and marks the slot pending until a compute
//    stream has waited for it; the copy stream carries nothing else, so the
//    copies of one call run back to back on the DMA engine;
//  - ensure(): hits refresh their age; each miss is copied into a slot that
//    this call does not name; a named expert whose copy is still pending (a
//    prefetch or a pin) is reported like a miss, so its compute runs after
//    wait();
//  - wait(): the compute stream waits for the ready events of every slot the
//    last ensure() named (completed events cost nothing), then, if copies
//    have changed the layer's device pointer table since the last wait,
//    uploads the table from its host mirror on that stream;
//  - release(): records, on the compute stream, the release event of those
//    slots; a later eviction of any of them waits for it. Until then pin and
//    prefetch leave those slots alone.
// With a NULL arena and pool the cache only keeps the books (no copies, no
// events): the policy can be simulated without a GPU.
#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "layer.h"

struct coli_expert_cache {
    coli_cache_cfg cfg;
    bool dry = false;
    std::vector<const uint8_t*> pools;             // [layer] host pool
    struct Slot {
        int32_t expert = -1;
        uint64_t last_use = 0;
        hipEvent_t ready = nullptr;       // after the copy that filled it
        hipEvent_t release = nullptr;     // after the compute that last read it
        bool release_recorded = false;
        bool pinned = false;              // never evicted while pinned
        bool pending = false;             // copy enqueued, no compute stream has waited for it
        bool prefetched = false;          // filled by a prefetch, not named by a call since
    };
    std::vector<std::vector<Slot>> slots;          // [layer][slot]
    std::vector<std::vector<int32_t>> where;       // [layer][expert] -> slot or -1
    std::vector<std::vector<int32_t>> used;        // [layer] slots named by the last ensure
    std::vector<char> open;                        // [layer] last ensure not yet released
    std::vector<std::vector<uint64_t>> usage;      // [layer][expert] lookups (history)
    std::vector<std::vector<double>> heat;         // [layer][expert] decaying session heat
    void** d_tables = nullptr;                     // device [layer][expert]
    uint8_t* h_slot_ptrs = nullptr;                // pinned: device address of every slot
    // host mirror of d_tables (updated by every copy), the pinned row each
    // upload reads, and the event after that upload (the row is rewritten
    // only once it has been read)
    std::vector<void*> h_tables;                   // [layer][expert]
    void** h_table_stage = nullptr;                // pinned [layer][expert]
    std::vector<hipEvent_t> table_done;            // [layer]
    std::vector<char> table_dirty, table_recorded; // [layer]
    uint64_t clock = 0;
    coli_cache_stats st{};
    // copy timing: ring of (start, stop) pairs, summed as they complete
    std::vector<std::pair<hipEvent_t, hipEvent_t>> timers;
    std::vector<bool> timer_live;
    size_t timer_next = 0;
    // pinned staging of the cached layer call, allocated by create: the
    // routing is read back through h_idx in chunks of kStagingIds entries;
    // h_phase holds the phase of every expert of every layer
    int32_t* h_idx = nullptr;          // [kStagingIds]
    uint8_t* h_phase = nullptr;        // [layer][expert]
};

namespace coli {

// Routing entries read back per chunk through the pinned staging buffer.
constexpr size_t kStagingIds = 16384;

// Host-forced copy failures (coli_debug_fail_copies): the next n copies fail
// before anything is enqueued.
static int32_t g_fail_copies = 0;

static coli_status harvest_timer(coli_expert_cache* c, size_t i, bool wait) {
    if (!c->timer_live[i]) return COLI_OK;
    if (wait) COLI_CHECK_HIP(hipEventSynchronize(c->timers[i].second));
    else if (hipEventQuery(c->timers[i].second) != hipSuccess) return COLI_OK;
    float ms = 0.f;
    COLI_CHECK_HIP(hipEventElapsedTime(&ms, c->timers[i].first, c->timers[i].second));
    c->st.copy_ns += (uint64_t)(ms * 1e6);
    c->timer_live[i] = false;
    return COLI_OK;
}

// Victim for a copy into `layer`: the first empty slot, else the least
// recently used slot (equal ages: the lowest expert id) among those that are
// not pinned and not excluded. -1 if there is none.
static int pick_victim(coli_expert_cache* c, int32_t layer, const std::vector<char>& excluded) {
    const auto& slots = c->slots[layer];
    int victim = -1;
    for (int s = 0; s < (int)slots.size(); ++s) {
        if (slots[s].pinned || excluded[s]) continue;
        if (slots[s].expert < 0) return s;
        if (victim < 0) { victim = s; continue; }
        const auto& a = slots[s];
        const auto& b = slots[victim];
        if (a.last_use < b.last_use || (a.last_use == b.last_use && a.expert < b.expert)) victim = s;
    }
    return victim;
}

// Slots an asynchronous pin or prefetch must not take: those named by a call
// that has not been released yet.
static std::vector<char> open_slots(coli_expert_cache* c, int32_t layer) {
    std::vector<char> ex(c->cfg.slots_per_layer, 0);
    if (c->open[layer])
        for (int32_t s : c->used[layer]) ex[s] = 1;
    return ex;
}

// Copy expert e of `layer` into slot `victim` (evicting its occupant). If a
// HIP call fails the error is returned with the slot left empty (its old
// occupant forgotten, e not resident) and the counters unchanged.
static coli_status load_slot(coli_expert_cache* c, int32_t layer, int32_t e, int victim,
                             uint64_t now) {
    const int S = c->cfg.slots_per_layer, E = c->cfg.n_experts;
    auto& sl = c->slots[layer][victim];
    const int32_t old = sl.expert;
    auto evict = [&]() {
        if (old >= 0) c->where[layer][old] = -1;
        sl.expert = -1;
        sl.prefetched = false;
        sl.pinned = false;
    };
    if (!c->dry) {
        auto failed = [&](hipError_t err, const char* what) {
            evict();
            sl.pending = false;
            return hip_fail(err, what);
        };
        if (g_fail_copies > 0) {
            --g_fail_copies;
            return failed(hipErrorOutOfMemory, "cache copy (host-forced failure)");
        }
        hipStream_t cs = (hipStream_t)c->cfg.copy_stream;
        const size_t bb = c->cfg.blob_bytes;
        uint8_t* dst = (uint8_t*)c->cfg.d_arena + ((size_t)layer * S + victim) * bb;
        const uint8_t* src = c->pools[layer] + (size_t)e * bb;
        hipError_t err;
        if (sl.release_recorded && (err = hipStreamWaitEvent(cs, sl.release, 0)) != hipSuccess)
            return failed(err, "cache copy: wait for the slot's release");
        const size_t ti = c->timer_next;
        coli_status hs = harvest_timer(c, ti, true);
        if (hs) {
            evict();
            return hs;
        }
        if ((err = hipEventRecord(c->timers[ti].first, cs)) != hipSuccess)
            return failed(err, "cache copy: timer start");
        if ((err = hipMemcpyAsync(dst, src, bb, hipMemcpyHostToDevice, cs)) != hipSuccess)
            return failed(err, "cache copy: hipMemcpyAsync");
        if ((err = hipEventRecord(c->timers[ti].second, cs)) != hipSuccess)
            return failed(err, "cache copy: timer stop");
        c->timer_next = (ti + 1) % c->timers.size();
        c->timer_live[ti] = true;
        // the expert's pointer goes to the host mirror of the layer's table;
        // wait() uploads it on the compute stream (a small copy here would
        // put a blit between the DMA copies of the copy stream)
        std::memcpy(&c->h_tables[(size_t)layer * E + e],
                    c->h_slot_ptrs + ((size_t)layer * S + victim) * sizeof(void*), sizeof(void*));
        c->table_dirty[layer] = 1;
        if ((err = hipEventRecord(sl.ready, cs)) != hipSuccess)
            return failed(err, "cache copy: ready event");
        sl.pending = true;
    }
    if (old >= 0) {
        c->where[layer][old] = -1;
        c->st.evictions++;
    }
    sl.expert = e;
    sl.last_use = now;
    sl.prefetched = false;
    c->where[layer][e] = victim;
    c->st.bytes_h2d += c->cfg.blob_bytes;
    return COLI_OK;
}

// Distinct ids of a request in first-appearance order; false if one is out of range.
static bool distinct_ids(const int32_t* ids, int32_t n, int32_t E, std::vector<int32_t>* out) {
    std::vector<char> seen(E, 0);
    out->clear();
    for (int32_t i = 0; i < n; ++i) {
        const int32_t e = ids[i];
        if (e < 0 || e >= E) return false;
        if (!seen[e]) { seen[e] = 1; out->push_back(e); }
    }
    return true;
}

// Make `ids` the pinned set of `layer`: earlier pins not in it become plain
// LRU entries; members not resident are copied in.
static coli_status pin_layer(coli_expert_cache* c, int32_t layer, const std::vector<int32_t>& ids) {
    const int S = c->cfg.slots_per_layer;
    auto& slots = c->slots[layer];
    auto& where = c->where[layer];
    if ((int)ids.size() > S) return fail(COLI_EBUSY, "cache_pin: more experts than slots");
    std::vector<char> excluded = open_slots(c, layer);
    std::vector<char> keep(S, 0);
    int need = 0;
    for (int32_t e : ids) {
        if (where[e] >= 0) keep[where[e]] = 1;
        else ++need;
    }
    int avail = 0;
    for (int s = 0; s < S; ++s) avail += !keep[s] && !excluded[s];
    if (need > avail) return fail(COLI_EBUSY, "cache_pin: not enough free slots (an unreleased call holds some)");
    for (int s = 0; s < S; ++s) slots[s].pinned = keep[s] != 0;
    const uint64_t now = ++c->clock;
    for (int32_t e : ids) {
        if (where[e] >= 0) continue;
        const int v = pick_victim(c, layer, excluded);
        if (v < 0) return fail(COLI_EBUSY, "cache_pin: no free slot");
        coli_status st = load_slot(c, layer, e, v, now);
        if (st) return st;
        slots[v].pinned = true;
        c->st.pin_loads++;
    }
    return COLI_OK;
}

coli_status cache_layer_table(coli_expert_cache* c, int32_t layer, int32_t n_experts,
                              const void* const** table) {
    if (!c || layer < 0 || layer >= c->cfg.n_layers) return fail(COLI_EINVAL, "cache: bad layer");
    if (n_experts != c->cfg.n_experts) return fail(COLI_EINVAL, "cache: expert count differs from the layer shape");
    if (c->dry) return fail(COLI_EINVAL, "cache: a bookkeeping-only cache has no device table");
    *table = (const void* const*)(c->d_tables + (size_t)layer * c->cfg.n_experts);
    return COLI_OK;
}

// Placement step of a cached layer call: read the routing back (blocking),
// make the selected experts of `layer` resident, and upload the phase of each
// selected expert (0: resident before the call, 1: copied by it) to d_phase.
// The experts named by d_idx [n] (entries < 0: slots dropped by top-p),
// read back to the host through the pinned staging in chunks (blocking).
static coli_status read_routing(coli_expert_cache* c, const int32_t* d_idx, int32_t n,
                                hipStream_t stream, std::vector<int32_t>* ids) {
    ids->clear();
    ids->reserve((size_t)n);
    for (size_t i0 = 0; i0 < (size_t)n; i0 += kStagingIds) {
        const size_t m = std::min(kStagingIds, (size_t)n - i0);
        COLI_CHECK_HIP(hipMemcpyAsync(c->h_idx, d_idx + i0, sizeof(int32_t) * m,
                                      hipMemcpyDeviceToHost, stream));
        COLI_CHECK_HIP(hipStreamSynchronize(stream));
        for (size_t i = 0; i < m; ++i)
            if (c->h_idx[i] >= 0) ids->push_back(c->h_idx[i]);
    }
    return COLI_OK;
}

coli_status cache_place(coli_expert_cache* c, int32_t layer, const int32_t* d_idx, int32_t n,
                        uint8_t* d_phase, int32_t* n_miss, hipStream_t stream) {
    if (c->dry) return fail(COLI_EINVAL, "cache: a bookkeeping-only cache cannot serve layer calls");
    std::vector<int32_t> ids;
    coli_status rs = read_routing(c, d_idx, n, stream, &ids);
    if (rs) return rs;
    std::vector<int32_t> miss(ids.size());
    coli_status st = coli_expert_cache_ensure(c, layer, ids.data(), (int32_t)ids.size(), miss.data());
    if (st) return st;
    uint8_t* ph = c->h_phase + (size_t)layer * c->cfg.n_experts;
    int32_t nm = 0;
    for (size_t i = 0; i < ids.size(); ++i) {
        ph[ids[i]] = miss[i] ? 1 : 0;
        nm += miss[i];
    }
    *n_miss = nm;
    // the previous upload from this layer's staging row finished before the
    // synchronisation above
    COLI_CHECK_HIP(hipMemcpyAsync(d_phase, ph, (size_t)c->cfg.n_experts, hipMemcpyHostToDevice, stream));
    return COLI_OK;
}

// Lookahead step: read back routing computed for `layer` from an earlier
// state (blocking) and prefetch the experts it names.
coli_status cache_prefetch_routed(coli_expert_cache* c, int32_t layer, const int32_t* d_idx,
                                  int32_t n, int32_t* started, hipStream_t stream) {
    if (c->dry) return fail(COLI_EINVAL, "cache: a bookkeeping-only cache cannot prefetch routed experts");
    std::vector<int32_t> ids;
    coli_status rs = read_routing(c, d_idx, n, stream, &ids);
    if (rs) return rs;
    return coli_expert_cache_prefetch(c, layer, ids.data(), (int32_t)ids.size(), started);
}

}  // namespace coli

using namespace coli;

extern "C" {

COLI_API coli_status coli_expert_cache_create(const coli_cache_cfg* cfg, struct coli_expert_cache** out) {
    try {
        if (!cfg || !out) return fail(COLI_EINVAL, "cache_create: NULL argument");
        if (cfg->n_layers <= 0 || cfg->n_experts <= 0 || cfg->n_experts > 1024 ||
            cfg->slots_per_layer <= 0 || cfg->blob_bytes == 0)
            return fail(COLI_EINVAL, "cache_create: bad sizes");
        const bool dry = cfg->d_arena == nullptr && cfg->h_pools == nullptr;
        if (!dry && (!cfg->d_arena || !cfg->h_pools))
            return fail(COLI_EINVAL, "cache_create: give both arena and pools, or neither");
        if (!dry)
            for (int l = 0; l < cfg->n_layers; ++l)
                if (!cfg->h_pools[l]) return fail(COLI_EINVAL, "cache_create: NULL pool pointer");
        auto* c = new coli_expert_cache();
        c->cfg = *cfg;
        c->cfg.h_pools = nullptr;
        c->dry = dry;
        if (!dry)
            for (int l = 0; l < cfg->n_layers; ++l) c->pools.push_back((const uint8_t*)cfg->h_pools[l]);
        const int L = cfg->n_layers, S = cfg->slots_per_layer, E = cfg->n_experts;
        c->slots.assign(L, std::vector<coli_expert_cache::Slot>(S));
        c->where.assign(L, std::vector<int32_t>(E, -1));
        c->used.assign(L, {});
        c->open.assign(L, 0);
        c->usage.assign(L, std::vector<uint64_t>(E, 0));
        c->heat.assign(L, std::vector<double>(E, 0.0));
        if (!dry) {
            auto cleanup = [&](coli_status code, const char* what) {
                coli_expert_cache_destroy(c);
                return fail(code, what);
            };
            if (hipMalloc((void**)&c->d_tables, sizeof(void*) * (size_t)L * E) != hipSuccess)
                return cleanup(COLI_EHIP, "cache_create: device table allocation failed");
            if (hipMemset(c->d_tables, 0, sizeof(void*) * (size_t)L * E) != hipSuccess)
                return cleanup(COLI_EHIP, "cache_create: device table clear failed");
            if (hipHostMalloc((void**)&c->h_slot_ptrs, sizeof(void*) * (size_t)L * S, hipHostMallocDefault) != hipSuccess)
                return cleanup(COLI_EHIP, "cache_create: pinned slot table allocation failed");
            for (int l = 0; l < L; ++l)
                for (int s = 0; s < S; ++s) {
                    void* p = (uint8_t*)cfg->d_arena + ((size_t)l * S + s) * cfg->blob_bytes;
                    std::memcpy(c->h_slot_ptrs + ((size_t)l * S + s) * sizeof(void*), &p, sizeof(void*));
                    auto& sl = c->slots[l][s];
                    if (hipEventCreateWithFlags(&sl.ready, hipEventDisableTiming) != hipSuccess ||
                        hipEventCreateWithFlags(&sl.release, hipEventDisableTiming) != hipSuccess)
                        return cleanup(COLI_EHIP, "cache_create: event creation failed");
                }
            if (hipHostMalloc((void**)&c->h_phase, (size_t)L * E, hipHostMallocDefault) != hipSuccess)
                return cleanup(COLI_EHIP, "cache_create: pinned phase table allocation failed");
            c->h_tables.assign((size_t)L * E, nullptr);
            c->table_dirty.assign(L, 0);
            c->table_recorded.assign(L, 0);
            c->table_done.assign(L, nullptr);
            if (hipHostMalloc((void**)&c->h_table_stage, sizeof(void*) * (size_t)L * E, hipHostMallocDefault) != hipSuccess)
                return cleanup(COLI_EHIP, "cache_create: pinned table staging allocation failed");
            for (int l = 0; l < L; ++l)
                if (hipEventCreateWithFlags(&c->table_done[l], hipEventDisableTiming) != hipSuccess)
                    return cleanup(COLI_EHIP, "cache_create: event creation failed");
            if (hipHostMalloc((void**)&c->h_idx, sizeof(int32_t) * kStagingIds, hipHostMallocDefault) != hipSuccess)
                return cleanup(COLI_EHIP, "cache_create: pinned routing staging allocation failed");
            std::memset(c->h_phase, 0, (size_t)L * E);
            c->timers.resize(64);
            c->timer_live.assign(64, false);
            for (auto& t : c->timers)
                if (hipEventCreate(&t.first) != hipSuccess || hipEventCreate(&t.second) != hipSuccess)
                    return cleanup(COLI_EHIP, "cache_create: event creation failed");
        }
        *out = c;
        return COLI_OK;
    } catch (const std::bad_alloc&) {
        return fail(COLI_ENOMEM, "cache_create: host allocation failed");
    }
}

COLI_API coli_status coli_debug_fail_copies(int32_t n) {
    if (n < 0) return fail(COLI_EINVAL, "debug_fail_copies: n must be >= 0");
    g_fail_copies = n;
    return COLI_OK;
}

COLI_API coli_status coli_expert_cache_destroy(struct coli_expert_cache* c) {
    if (!c) return COLI_OK;
    if (!c->dry) (void)hipDeviceSynchronize();
    for (auto& layer : c->slots)
        for (auto& s : layer) {
            if (s.ready) (void)hipEventDestroy(s.ready);
            if (s.release) (void)hipEventDestroy(s.release);
        }
    for (auto& t : c->timers) {
        if (t.first) (void)hipEventDestroy(t.first);
        if (t.second) (void)hipEventDestroy(t.second);
    }
    for (hipEvent_t ev : c->table_done)
        if (ev) (void)hipEventDestroy(ev);
    if (c->d_tables) (void)hipFree(c->d_tables);
    if (c->h_slot_ptrs) (void)hipHostFree(c->h_slot_ptrs);
    if (c->h_table_stage) (void)hipHostFree(c->h_table_stage);
    if (c->h_idx) (void)hipHostFree(c->h_idx);
    if (c->h_phase) (void)hipHostFree(c->h_phase);
    delete c;
    return COLI_OK;
}

COLI_API coli_status coli_expert_cache_ensure(struct coli_expert_cache* c, int32_t layer,
                                              const int32_t* h_ids, int32_t n, int32_t* h_miss_mask) {
    try {
        if (!c || layer < 0 || layer >= c->cfg.n_layers || n < 0 || (n > 0 && !h_ids))
            return fail(COLI_EINVAL, "cache_ensure: bad arguments");
        const int S = c->cfg.slots_per_layer, E = c->cfg.n_experts;
        auto& slots = c->slots[layer];
        auto& where = c->where[layer];
        // distinct ids of this call, in first-appearance order
        std::vector<int32_t> ids;
        if (!distinct_ids(h_ids, n, E, &ids)) return fail(COLI_EINVAL, "cache_ensure: expert id out of range");
        if ((int)ids.size() > S) return fail(COLI_EBUSY, "cache_ensure: more distinct experts than slots");
        // capacity first, so that a refused call changes nothing
        std::vector<char> named(S, 0);
        std::vector<int32_t> misses;
        for (int32_t e : ids) {
            if (where[e] >= 0) named[where[e]] = 1;
            else misses.push_back(e);
        }
        int avail = 0;
        for (int s = 0; s < S; ++s) avail += !named[s] && !slots[s].pinned;
        if ((int)misses.size() > avail)
            return fail(COLI_EBUSY, "cache_ensure: more unpinned experts than unpinned slots");
        const uint64_t now = ++c->clock;
        std::vector<char> late(E, 0);          // compute after wait(): copied or still pending
        std::vector<int32_t> used;
        for (int32_t e : ids) {
            c->usage[layer][e] += 1;
            c->heat[layer][e] += 1.0;
            const int32_t s = where[e];
            if (s < 0) continue;
            auto& sl = slots[s];
            sl.last_use = now;
            c->st.hits++;
            if (sl.pinned) c->st.pin_hits++;
            if (sl.prefetched) { c->st.prefetch_hits++; sl.prefetched = false; }
            if (sl.pending) late[e] = 1;
            used.push_back(s);
        }
        c->st.lookups += ids.size();
        for (int32_t e : misses) {
            const int v = pick_victim(c, layer, named);
            if (v < 0) return fail(COLI_EBUSY, "cache_ensure: no free slot");
            coli_status st = load_slot(c, layer, e, v, now);
            if (st) return st;
            named[v] = 1;
            late[e] = 1;
            used.push_back(v);
            c->st.misses++;
        }
        c->used[layer] = used;
        c->open[layer] = 1;
        if (h_miss_mask)
            for (int32_t i = 0; i < n; ++i) h_miss_mask[i] = late[h_ids[i]];
        return COLI_OK;
    } catch (const std::bad_alloc&) {
        return fail(COLI_ENOMEM, "cache_ensure: host allocation failed");
    }
}

COLI_API coli_status coli_expert_cache_wait(struct coli_expert_cache* c, int32_t layer, void* stream) {
    if (!c || layer < 0 || layer >= c->cfg.n_layers) return fail(COLI_EINVAL, "cache_wait: bad arguments");
    if (c->dry) return COLI_OK;
    for (int32_t s : c->used[layer]) {
        COLI_CHECK_HIP(hipStreamWaitEvent((hipStream_t)stream, c->slots[layer][s].ready, 0));
        c->slots[layer][s].pending = false;
    }
    if (c->table_dirty[layer]) {
        const size_t E = (size_t)c->cfg.n_experts;
        void** row = c->h_table_stage + (size_t)layer * E;
        if (c->table_recorded[layer]) COLI_CHECK_HIP(hipEventSynchronize(c->table_done[layer]));
        std::memcpy(row, &c->h_tables[(size_t)layer * E], E * sizeof(void*));
        COLI_CHECK_HIP(hipMemcpyAsync(c->d_tables + (size_t)layer * E, row, E * sizeof(void*),
                                      hipMemcpyHostToDevice, (hipStream_t)stream));
        COLI_CHECK_HIP(hipEventRecord(c->table_done[layer], (hipStream_t)stream));
        c->table_recorded[layer] = 1;
        c->table_dirty[layer] = 0;
    }
    return COLI_OK;
}

COLI_API coli_status coli_expert_cache_release(struct coli_expert_cache* c, int32_t layer, void* stream) {
    if (!c || layer < 0 || layer >= c->cfg.n_layers) return fail(COLI_EINVAL, "cache_release: bad arguments");
    c->open[layer] = 0;
    if (c->dry) return COLI_OK;
    for (int32_t s : c->used[layer]) {
        auto& sl = c->slots[layer][s];
        COLI_CHECK_HIP(hipEventRecord(sl.release, (hipStream_t)stream));
        sl.release_recorded = true;
    }
    return COLI_OK;
}

COLI_API coli_status coli_expert_cache_table(struct coli_expert_cache* c, int32_t layer,
                                             const void* const** d_table) {
    if (!c || !d_table) return fail(COLI_EINVAL, "cache_table: NULL argument");
    return cache_layer_table(c, layer, c->cfg.n_experts, d_table);
}

COLI_API coli_status coli_expert_cache_stats(struct coli_expert_cache* c, coli_cache_stats* out) {
    if (!c || !out) return fail(COLI_EINVAL, "cache_stats: NULL argument");
    for (size_t i = 0; i < c->timers.size(); ++i) {
        coli_status s = harvest_timer(c, i, true);
        if (s) return s;
    }
    *out = c->st;
    return COLI_OK;
}

COLI_API coli_status coli_expert_cache_reset(struct coli_expert_cache* c) {
    if (!c) return fail(COLI_EINVAL, "cache_reset: NULL argument");
    if (!c->dry) COLI_CHECK_HIP(hipStreamSynchronize((hipStream_t)c->cfg.copy_stream));
    for (auto& layer : c->slots)
        for (auto& s : layer) {
            s.expert = -1;
            s.last_use = 0;
            s.pinned = s.pending = s.prefetched = false;
        }
    for (auto& w : c->where) std::fill(w.begin(), w.end(), -1);
    for (auto& u : c->used) u.clear();
    std::fill(c->open.begin(), c->open.end(), 0);
    for (auto& u : c->usage) std::fill(u.begin(), u.end(), 0);
    for (auto& h : c->heat) std::fill(h.begin(), h.end(), 0.0);
    c->clock = 0;
    for (size_t i = 0; i < c->timer_live.size(); ++i) c->timer_live[i] = false;
    c->st = coli_cache_stats{};
    return COLI_OK;
}

COLI_API coli_status coli_expert_cache_pin(struct coli_expert_cache* c, int32_t layer,
                                           const int32_t* h_ids, int32_t n) {
    try {
        if (!c || layer < 0 || layer >= c->cfg.n_layers || n < 0 || (n > 0 && !h_ids))
            return fail(COLI_EINVAL, "cache_pin: bad arguments");
        std::vector<int32_t> ids;
        if (!distinct_ids(h_ids, n, c->cfg.n_experts, &ids))
            return fail(COLI_EINVAL, "cache_pin: expert id out of range");
        return pin_layer(c, layer, ids);
    } catch (const std::bad_alloc&) {
        return fail(COLI_ENOMEM, "cache_pin: host allocation failed");
    }
}

COLI_API coli_status coli_expert_cache_usage(struct coli_expert_cache* c, uint64_t* h_counts) {
    if (!c || !h_counts) return fail(COLI_EINVAL, "cache_usage: NULL argument");
    const size_t E = (size_t)c->cfg.n_experts;
    for (size_t l = 0; l < c->usage.size(); ++l)
        std::memcpy(h_counts + l * E, c->usage[l].data(), E * sizeof(uint64_t));
    return COLI_OK;
}

COLI_API coli_status coli_expert_cache_pin_hot(struct coli_expert_cache* c, const uint64_t* h_counts,
                                               int32_t per_layer) {
    try {
        if (!c) return fail(COLI_EINVAL, "cache_pin_hot: NULL cache");
        if (per_layer < 0 || per_layer > c->cfg.slots_per_layer)
            return fail(COLI_EINVAL, "cache_pin_hot: per_layer must be in [0, slots_per_layer]");
        const int L = c->cfg.n_layers, E = c->cfg.n_experts;
        for (int l = 0; l < L; ++l) {
            const uint64_t* cnt = h_counts ? h_counts + (size_t)l * E : c->usage[l].data();
            std::vector<int32_t> order(E);
            for (int e = 0; e < E; ++e) order[e] = e;
            std::stable_sort(order.begin(), order.end(),
                             [cnt](int32_t a, int32_t b) { return cnt[a] > cnt[b]; });
            std::vector<int32_t> ids;
            for (int i = 0; i < E && (int)ids.size() < per_layer; ++i)
                if (cnt[order[i]] > 0) ids.push_back(order[i]);
            coli_status st = pin_layer(c, l, ids);
            if (st) return st;
        }
        return COLI_OK;
    } catch (const std::bad_alloc&) {
        return fail(COLI_ENOMEM, "cache_pin_hot: host allocation failed");
    }
}

COLI_API coli_status coli_expert_cache_repin(struct coli_expert_cache* c, int32_t max_swaps,
                                             float hysteresis, float decay, int32_t* h_swaps) {
    try {
        if (!c || max_swaps < 0 || !(hysteresis >= 0.f) || !(decay >= 0.f && decay <= 1.f))
            return fail(COLI_EINVAL, "cache_repin: bad arguments");
        const int L = c->cfg.n_layers, E = c->cfg.n_experts;
        int32_t swaps = 0;
        for (int l = 0; l < L; ++l) {
            auto& slots = c->slots[l];
            auto& where = c->where[l];
            const auto& heat = c->heat[l];
            std::vector<char> excluded = open_slots(c, l);
            for (int n = 0; n < max_swaps; ++n) {
                // coldest pinned expert (equal heat: the higher id leaves first)
                int cold = -1;
                for (const auto& sl : slots)
                    if (sl.pinned && (cold < 0 || heat[sl.expert] < heat[cold] ||
                                      (heat[sl.expert] == heat[cold] && sl.expert > cold)))
                        cold = sl.expert;
                // hottest expert that is not pinned (equal heat: the lower id)
                int hot = -1;
                for (int e = 0; e < E; ++e) {
                    if (where[e] >= 0 && slots[where[e]].pinned) continue;
                    if (heat[e] > 0.0 && (hot < 0 || heat[e] > heat[hot])) hot = e;
                }
                if (cold < 0 || hot < 0) break;
                if (!(heat[hot] > (1.0 + (double)hysteresis) * heat[cold])) break;
                slots[where[cold]].pinned = false;          // stays resident as an LRU entry
                if (where[hot] >= 0) {
                    slots[where[hot]].pinned = true;
                } else {
                    const int v = pick_victim(c, l, excluded);
                    if (v < 0) { slots[where[cold]].pinned = true; break; }
                    coli_status st = load_slot(c, l, hot, v, ++c->clock);
                    if (st) return st;
                    slots[v].pinned = true;
                    c->st.pin_loads++;
                }
                ++swaps;
            }
        }
        for (auto& h : c->heat)
            for (double& v : h) v *= (double)decay;
        c->st.repin_swaps += (uint64_t)swaps;
        if (h_swaps) *h_swaps = swaps;
        return COLI_OK;
    } catch (const std::bad_alloc&) {
        return fail(COLI_ENOMEM, "cache_repin: host allocation failed");
    }
}

COLI_API coli_status coli_expert_cache_prefetch(struct coli_expert_cache* c, int32_t layer,
                                                const int32_t* h_ids, int32_t n,
                                                int32_t* h_started) {
    try {
        if (!c || layer < 0 || layer >= c->cfg.n_layers || n < 0 || (n > 0 && !h_ids))
            return fail(COLI_EINVAL, "cache_prefetch: bad arguments");
        std::vector<int32_t> ids;
        if (!distinct_ids(h_ids, n, c->cfg.n_experts, &ids))
            return fail(COLI_EINVAL, "cache_prefetch: expert id out of range");
        std::vector<char> excluded = open_slots(c, layer);
        // experts already resident (or in flight) are not read again and keep
        // their slots for this request
        for (int32_t e : ids)
            if (c->where[layer][e] >= 0) excluded[c->where[layer][e]] = 1;
        const uint64_t now = ++c->clock;
        int32_t started = 0;
        for (int32_t e : ids) {
            if (c->where[layer][e] >= 0) continue;
            const int v = pick_victim(c, layer, excluded);
            if (v < 0) break;
            coli_status st = load_slot(c, layer, e, v, now);
            if (st) return st;
            c->slots[layer][v].prefetched = true;
            excluded[v] = 1;
            c->st.prefetches++;
            ++started;
        }
        if (h_started) *h_started = started;
        return COLI_OK;
    } catch (const std::bad_alloc&) {
        return fail(COLI_ENOMEM, "cache_prefetch: host allocation failed");
    }
}

}  // extern "C"
