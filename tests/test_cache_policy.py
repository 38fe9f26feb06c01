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
