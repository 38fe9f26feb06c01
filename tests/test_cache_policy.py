"""The expert cache's placement policy, simulated without a GPU (a cache with no
arena and no pool keeps only the books), against an independent LRU model:
per layer, hits refresh their age, a miss takes an empty slot if any, else the
least recently used slot that the same call does not use (practical guide
section 二: per-layer LRU; one read per miss; a request for an expert already
being read is not read again)."""
import numpy as np
import pytest

import int4_routed_expert_sigmoid_amd as coli
import synth


class LruModel:
    def __init__(self, n_layers, slots):
        self.slots = slots
        self.res = [dict() for _ in range(n_layers)]     # expert -> last use
        self.clock = 0
        self.hits = self.misses = self.evictions = 0

    def ensure(self, layer, ids):
        self.clock += 1
        res = self.res[layer]
        distinct = list(dict.fromkeys(int(e) for e in ids))
        if len(distinct) > self.slots:
            raise OverflowError
        miss_set = [e for e in distinct if e not in res]
        for e in distinct:
            if e in res:
                res[e] = self.clock
                self.hits += 1
        for e in miss_set:
            if len(res) >= self.slots:
                victims = [(t, x) for x, t in res.items() if x not in distinct]
                _, v = min(victims)
                del res[v]
                self.evictions += 1
            res[e] = self.clock
            self.misses += 1
        return np.array([1 if e in miss_set else 0 for e in ids], dtype=np.int32)


def _cache(n_layers, n_experts, slots):
    return coli.ExpertCache(n_layers, n_experts, slots, 18_915_328)


def test_matches_lru_model_on_locality_routing():
    L, E, k, S, T = 3, 256, 8, 24, 300
    c = _cache(L, E, S)
    m = LruModel(L, S)
    for layer in range(L):
        _, chosen = synth.locality_logits(5, layer, T, E, k, keep_p=0.6)
        for t in range(T):
            got = c.ensure(layer, chosen[t])
            ref = m.ensure(layer, chosen[t])
            assert np.array_equal(got, ref), (layer, t)
    st = c.stats()
    assert (st["hits"], st["misses"], st["evictions"]) == (m.hits, m.misses, m.evictions)
    assert st["bytes_h2d"] == m.misses * 18_915_328
    assert st["lookups"] == L * T * k
    assert m.hits > 0 and m.evictions > 0


def test_capacity_equal_to_k_evicts_every_new_expert():
    c = _cache(1, 16, 4)
    m = LruModel(1, 4)
    rng = np.random.default_rng(0)
    for _ in range(200):
        ids = rng.choice(16, size=4, replace=False)
        assert np.array_equal(c.ensure(0, ids), m.ensure(0, ids))
    assert c.stats()["evictions"] == m.evictions


def test_duplicates_count_once_and_errors():
    c = _cache(2, 8, 3)
    miss = c.ensure(1, [5, 5, 2])
    assert miss.tolist() == [1, 1, 1]
    st = c.stats()
    assert st["misses"] == 2 and st["lookups"] == 2
    assert c.ensure(1, [2, 5]).tolist() == [0, 0]
    with pytest.raises(coli.ColiError) as ei:
        c.ensure(1, [0, 1, 2, 3])
    assert ei.value.code == coli.COLI_EBUSY
    with pytest.raises(coli.ColiError):
        c.ensure(1, [9])
    with pytest.raises(coli.ColiError):
        c.ensure(2, [0])
    c.reset()
    assert c.stats()["misses"] == 0
    assert c.ensure(1, [2]).tolist() == [1]


def test_layers_are_independent():
    c = _cache(2, 8, 2)
    c.ensure(0, [1, 2])
    assert c.ensure(1, [1, 2]).tolist() == [1, 1]
    assert c.ensure(0, [1, 2]).tolist() == [0, 0]


def test_bookkeeping_cache_has_no_device_table():
    c = _cache(1, 8, 2)
    with pytest.raises(coli.ColiError):
        c.table_ptr(0)


# ----------------------------------------------------- learned placement
class PlacementModel:
    """Independent model of the learned placement (practical guide section 五:
    usage history, pinned experts sharing the layer's slots with the LRU,
    pin-the-hottest, repin from a decaying heat map with hysteresis and a swap
    limit; section 二: lookahead prefetch). Residency is a dict per layer."""

    def __init__(self, L, E, S):
        self.E, self.S = E, S
        self.res = [dict() for _ in range(L)]        # expert -> [last_use, pinned, prefetched]
        self.open = [set() for _ in range(L)]        # experts named by an unreleased call
        self.usage = np.zeros((L, E), np.uint64)
        self.heat = np.zeros((L, E), np.float64)
        self.clock = 0
        self.st = dict(hits=0, misses=0, evictions=0, lookups=0, pin_hits=0, pin_loads=0,
                       prefetches=0, prefetch_hits=0, repin_swaps=0)

    def _victim(self, layer, excluded):
        res = self.res[layer]
        if len(res) < self.S:
            return None                               # an empty slot
        cand = [(v[0], e) for e, v in res.items() if not v[1] and e not in excluded]
        if not cand:
            raise OverflowError
        return min(cand)[1]

    def _load(self, layer, e, excluded, now):
        v = self._victim(layer, excluded)
        if v is not None:
            del self.res[layer][v]
            self.st["evictions"] += 1
        self.res[layer][e] = [now, False, False]

    def ensure(self, layer, ids):
        res = self.res[layer]
        d = list(dict.fromkeys(int(e) for e in ids))
        if len(d) > self.S:
            raise OverflowError
        hits = [e for e in d if e in res]
        misses = [e for e in d if e not in res]
        free = self.S - len(hits) - sum(1 for e, v in res.items() if v[1] and e not in hits)
        if len(misses) > free:
            raise OverflowError
        self.clock += 1
        for e in d:
            self.usage[layer, e] += 1
            self.heat[layer, e] += 1.0
        for e in hits:
            res[e][0] = self.clock
            self.st["hits"] += 1
            self.st["pin_hits"] += res[e][1]
            if res[e][2]:
                self.st["prefetch_hits"] += 1
                res[e][2] = False
        self.st["lookups"] += len(d)
        for e in misses:
            self._load(layer, e, set(d), self.clock)
            self.st["misses"] += 1
        self.open[layer] = set(d)
        return np.array([1 if e in misses else 0 for e in ids], np.int32)

    def release(self, layer):
        self.open[layer] = set()

    def pin(self, layer, ids):
        res = self.res[layer]
        d = list(dict.fromkeys(int(e) for e in ids))
        need = [e for e in d if e not in res]
        excluded = self.open[layer]
        avail = self.S - sum(1 for e in res if e in d) - sum(1 for e in excluded if e not in d)
        if len(d) > self.S or len(need) > avail:
            raise OverflowError
        for e, v in res.items():
            v[1] = e in d
        self.clock += 1
        for e in need:
            self._load(layer, e, excluded, self.clock)
            res[e][1] = True
            self.st["pin_loads"] += 1

    def pin_hot(self, per_layer, counts=None):
        counts = self.usage if counts is None else counts
        for layer in range(len(self.res)):
            order = sorted(range(self.E), key=lambda e: (-int(counts[layer, e]), e))
            self.pin(layer, [e for e in order if counts[layer, e] > 0][:per_layer])

    def repin(self, max_swaps, hyst, decay):
        total = 0
        for layer, res in enumerate(self.res):
            h = self.heat[layer]
            for _ in range(max_swaps):
                pinned = [e for e, v in res.items() if v[1]]
                if not pinned:
                    break
                cold = min(pinned, key=lambda e: (h[e], -e))
                cand = [e for e in range(self.E) if not (e in res and res[e][1]) and h[e] > 0]
                if not cand:
                    break
                hot = min(cand, key=lambda e: (-h[e], e))
                if not h[hot] > (1.0 + hyst) * h[cold]:
                    break
                res[cold][1] = False
                if hot in res:
                    res[hot][1] = True
                else:
                    try:
                        self.clock += 1
                        self._load(layer, hot, self.open[layer], self.clock)
                    except OverflowError:
                        res[cold][1] = True
                        break
                    res[hot][1] = True
                    self.st["pin_loads"] += 1
                total += 1
        self.heat *= decay
        self.st["repin_swaps"] += total
        return total

    def prefetch(self, layer, ids):
        res = self.res[layer]
        d = list(dict.fromkeys(int(e) for e in ids))
        excluded = set(self.open[layer]) | {e for e in d if e in res}
        self.clock += 1
        n = 0
        for e in d:
            if e in res:
                continue
            try:
                self._load(layer, e, excluded, self.clock)
            except OverflowError:
                break
            res[e][2] = True
            excluded.add(e)
            self.st["prefetches"] += 1
            n += 1
        return n


def _same_stats(c, m):
    st = c.stats()
    for key, v in m.st.items():
        assert st[key] == v, (key, st[key], v)


def test_learned_placement_matches_model():
    L, E, k, S, T = 2, 64, 8, 20, 400
    c = _cache(L, E, S)
    m = PlacementModel(L, E, S)
    rng = np.random.default_rng(3)
    chosen = [synth.locality_logits(9, l, T, E, k, keep_p=0.6)[1] for l in range(L)]
    for t in range(T):
        for layer in range(L):
            if t == 100 and layer == 0:
                c.pin_hot(6)
                m.pin_hot(6)
            if t > 0 and t % 50 == 0 and layer == 0:
                assert c.repin(4, 0.25, 0.5) == m.repin(4, 0.25, 0.5)
            if t % 3 == 0:
                # lookahead of this token's picks, partly wrong
                guess = [e if rng.random() < 0.7 else int(rng.integers(E)) for e in chosen[layer][t]]
                assert c.prefetch(layer, guess) == m.prefetch(layer, guess)
            assert np.array_equal(c.ensure(layer, chosen[layer][t]), m.ensure(layer, chosen[layer][t]))
            if t % 7 == 0:
                # a pin between ensure and release must leave the call's slots alone
                hot = np.argsort(-m.usage[layer].astype(np.int64), kind="stable")[:3]
                c.pin(layer, hot)
                m.pin(layer, hot)
            c.release(layer)
            m.release(layer)
        _same_stats(c, m)
    assert np.array_equal(c.usage(), m.usage)
    st = c.stats()
    assert st["pin_hits"] > 0 and st["prefetch_hits"] > 0 and st["repin_swaps"] > 0
    assert st["bytes_h2d"] == (st["misses"] + st["pin_loads"] + st["prefetches"]) * 18_915_328


def test_usage_history_counts_calls():
    c = _cache(2, 8, 4)
    calls = [(0, [1, 2, 2]), (0, [2, 3]), (1, [7]), (0, [1])]
    for layer, ids in calls:
        c.ensure(layer, ids)
        c.release(layer)
    ref = np.zeros((2, 8), np.uint64)
    ref[0, 1], ref[0, 2], ref[0, 3], ref[1, 7] = 2, 2, 1, 1
    assert np.array_equal(c.usage(), ref)


def test_pinned_experts_survive_churn():
    c = _cache(1, 32, 4)
    c.pin(0, [5, 9])
    assert c.stats()["pin_loads"] == 2
    for i in range(40):
        ids = [10 + i % 20, 10 + (i + 7) % 20]
        c.ensure(0, ids)
        c.release(0)
    assert c.ensure(0, [5, 9]).tolist() == [0, 0]
    assert c.stats()["pin_hits"] == 2


def test_pins_limit_a_call_and_refusal_changes_nothing():
    c = _cache(1, 16, 4)
    c.pin(0, [0, 1, 2])
    c.ensure(0, [3])                                   # one unpinned slot left
    c.release(0)
    before = c.stats()
    with pytest.raises(coli.ColiError) as ei:
        c.ensure(0, [4, 5])
    assert ei.value.code == coli.COLI_EBUSY
    assert c.stats() == before
    assert c.ensure(0, [3, 0]).tolist() == [0, 0]     # still resident
    c.release(0)
    with pytest.raises(coli.ColiError):
        c.pin(0, [0, 1, 2, 3, 4])                      # more than the slots
    c.pin(0, [])                                       # unpin all
    assert c.ensure(0, [4, 5, 6]).tolist() == [1, 1, 1]


def test_pin_hot_takes_the_hottest_from_a_history():
    c = _cache(2, 8, 4)
    counts = np.zeros((2, 8), np.uint64)
    counts[0] = [5, 0, 9, 9, 1, 0, 0, 2]
    counts[1] = [0, 0, 0, 0, 0, 0, 0, 3]
    c.pin_hot(3, counts)
    st = c.stats()
    assert st["pin_loads"] == 3 + 1                    # layer 1 has one expert with count > 0
    # layer 0 pinned {2, 3, 0}: they survive a churn of other experts
    for ids in ([1], [4], [5], [6], [7], [1]):
        c.ensure(0, ids)
        c.release(0)
    assert c.ensure(0, [2, 3, 0]).tolist() == [0, 0, 0]
    with pytest.raises(coli.ColiError):
        c.pin_hot(5)                                   # more than the slots


def test_repin_hysteresis_and_swap_limit():
    c = _cache(1, 16, 8)
    c.pin(0, [0])
    for _ in range(4):                                 # heat 4 on the pinned expert
        c.ensure(0, [0])
        c.release(0)
    for _ in range(5):                                 # heat 5 < 1.25 * 4
        c.ensure(0, [1])
        c.release(0)
    assert c.repin(4, 0.25, 1.0) == 0
    c.ensure(0, [1])                                   # heat 6 > 5
    c.release(0)
    assert c.repin(4, 0.25, 1.0) == 1
    assert c.stats()["repin_swaps"] == 1
    # six pinned cold experts against seven hot ones: at most four swaps per call
    c2 = _cache(1, 16, 16)
    c2.pin(0, [0, 1, 2, 3, 4, 5])
    for e in range(6, 13):
        for _ in range(3):
            c2.ensure(0, [e])
            c2.release(0)
    assert c2.repin(4, 0.25, 0.5) == 4
    assert c2.repin(4, 0.25, 0.5) == 2
    assert c2.repin(4, 0.25, 0.5) == 0


def test_prefetch_skips_resident_pinned_and_open():
    c = _cache(1, 16, 4)
    c.pin(0, [0])
    c.ensure(0, [1, 2])                                # open call holds 1 and 2
    assert c.prefetch(0, [0, 1, 3, 4, 5]) == 1         # only one free slot (3 taken, then none)
    c.release(0)
    assert c.prefetch(0, [4]) == 1                     # now the LRU (1) may go
    assert c.ensure(0, [3, 4]).tolist() == [0, 0]
    st = c.stats()
    assert st["prefetches"] == 2 and st["prefetch_hits"] == 2
