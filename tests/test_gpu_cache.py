"""Cached layer calls vs resident ones (practical guide section 二: placement
decides speed only, never routing or precision). Experts of several layers
live in pinned host memory; a small HBM cache per layer holds the resident
ones; the outputs must be bit-identical to calls with every expert resident."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import ExpertSet, rel_l2_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def coli():
    import int4_routed_expert_sigmoid_amd as c
    c.lib()
    return c


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _setup(coli, L, H, I, E, k, group, slots):
    import torch
    shape = coli.MoEShape(H, I, E, 1, k, group)
    _, nbytes = coli.blob_layout(shape)
    sets = [ExpertSet(coli, shape, seed=40 + l, layer=l) for l in range(L)]
    pool = torch.empty(L * E * nbytes, dtype=torch.uint8).pin_memory()
    for l, s in enumerate(sets):
        for e in range(E):
            pool[(l * E + e) * nbytes:(l * E + e + 1) * nbytes].copy_(s.blobs[e].cpu())
    arena = torch.zeros(L * slots * nbytes, dtype=torch.uint8, device="cuda")
    copy_stream = torch.cuda.Stream()
    cache = coli.ExpertCache(L, E, slots, nbytes, arena=arena, pools=pool, copy_stream=copy_stream)
    return shape, sets, cache


@pytest.mark.parametrize("T,group", [(1, 0), (8, 64), (20, 0)])
def test_cached_equals_resident(coli, T, group):
    import torch
    L, H, I, k, steps = 3, 512, 256, 4, 12
    E = 32 if T == 1 else 64
    slots = max(10, min(E, T * k))        # a call may name up to T*k distinct experts
    shape, sets, cache = _setup(coli, L, H, I, E, k, group, slots)
    ws_c = coli.workspace(shape, T)
    ws_r = coli.workspace(shape, T)
    for step in range(steps):
        for l in range(L):
            lg, _ = synth.locality_logits(50 + l, l, steps * T, E, k, keep_p=0.6)
            lgs = lg[step * T:(step + 1) * T]
            x = synth.activations(50, l, step * T, T, H)
            yc = coli.layer_fwd(shape, _dev(x), shared_blob=sets[l].shared_blob, logits=_dev(lgs),
                                cache=cache, layer=l, ws=ws_c)
            yr = coli.layer_fwd(shape, _dev(x), table=sets[l].table, shared_blob=sets[l].shared_blob,
                                logits=_dev(lgs), ws=ws_r)
            torch.cuda.synchronize()
            assert np.array_equal(yc.cpu().numpy(), yr.cpu().numpy()), (step, l)
    st = cache.stats()
    assert st["misses"] > 0 and st["hits"] > 0
    assert st["bytes_h2d"] == st["misses"] * coli.blob_layout(shape)[1]
    assert st["copy_ns"] > 0
    # and the cached result is the layer: spot-check the last call against the oracle
    _, y64, _, _ = oracle.layer(x, sets[L - 1].oracle_list(), sets[L - 1].shared_oracle, k, group,
                                1.0, logits=lgs)
    tol = 1e-3 if T <= 16 else 2e-2
    assert rel_l2_rows(yc.cpu().numpy(), y64).max() <= tol
    cache.close()


def test_slots_equal_top_k(coli):
    """Every new expert evicts: the smallest legal cache."""
    import torch
    L, H, I, E, k = 1, 256, 128, 16, 4
    shape, sets, cache = _setup(coli, L, H, I, E, k, 0, k)
    ws = coli.workspace(shape, 1)
    lg = synth.zipf_logits(60, 0, 0, 30, E, s=0.5)
    x = synth.activations(60, 0, 0, 30, H)
    for t in range(30):
        yc = coli.layer_fwd(shape, _dev(x[t:t + 1]), shared_blob=sets[0].shared_blob,
                            logits=_dev(lg[t:t + 1]), cache=cache, layer=0, ws=ws)
        yr = coli.layer_fwd(shape, _dev(x[t:t + 1]), table=sets[0].table,
                            shared_blob=sets[0].shared_blob, logits=_dev(lg[t:t + 1]))
        torch.cuda.synchronize()
        assert np.array_equal(yc.cpu().numpy(), yr.cpu().numpy()), t
    st = cache.stats()
    assert st["evictions"] > 0
    cache.close()


@pytest.mark.parametrize("T", [1, 8, 20])
def test_learned_placement_equals_resident(coli, T):
    """Pins (from the cache's own usage history), repins and lookahead prefetches
    change which experts are resident and when they are copied, never the
    output: every cached call equals the resident call bit for bit. The
    lookahead is run right before each call with the call's own routing input,
    so the call finds its experts prefetched with copies possibly in flight."""
    import torch
    L, H, I, k, steps = 2, 512, 256, 4, 10
    E = 32 if T == 1 else 64
    # room for the largest call (at most 4, 15 and 23 distinct experts for the
    # three cases with these seeds) next to 4 pinned experts, with evictions
    slots = {1: 12, 8: 24, 20: 32}[T]
    shape, sets, cache = _setup(coli, L, H, I, E, k, 0, slots)
    ws_c = coli.workspace(shape, T)
    ws_r = coli.workspace(shape, T)
    started = 0
    for step in range(steps):
        if step == 3:
            cache.pin_hot(4)
        if step >= 4 and step % 2 == 0:
            cache.repin(4, 0.25, 0.5)
        for l in range(L):
            lg, _ = synth.locality_logits(90 + l, l, steps * T, E, k, keep_p=0.6)
            lgs = _dev(lg[step * T:(step + 1) * T])
            x = _dev(synth.activations(90, l, step * T, T, H))
            if step % 2 == 1:
                started += coli.lookahead(shape, x, cache, l, logits=lgs, ws=ws_c)
            yc = coli.layer_fwd(shape, x, shared_blob=sets[l].shared_blob, logits=lgs,
                                cache=cache, layer=l, ws=ws_c)
            yr = coli.layer_fwd(shape, x, table=sets[l].table, shared_blob=sets[l].shared_blob,
                                logits=lgs, ws=ws_r)
            torch.cuda.synchronize()
            assert np.array_equal(yc.cpu().numpy(), yr.cpu().numpy()), (step, l)
    st = cache.stats()
    assert started > 0 and st["prefetches"] == started and st["prefetch_hits"] > 0
    assert st["pin_loads"] + st["pin_hits"] > 0
    assert st["bytes_h2d"] == (st["misses"] + st["pin_loads"] + st["prefetches"]) * \
        coli.blob_layout(shape)[1]
    cache.close()


def test_lookahead_with_router(coli):
    """The lookahead's own routing (router weights applied to a state) prefetches
    exactly what the layer call with the same state and router then names."""
    import torch
    L, H, I, E, k, T = 1, 512, 256, 32, 4, 3
    shape, sets, cache = _setup(coli, L, H, I, E, k, 0, 16)
    wr = synth.router_weights(95, 0, E, H)
    b = synth.bias(95, 0, E)
    x = synth.activations(95, 0, 0, T, H)
    ws = coli.workspace(shape, T)
    n = coli.lookahead(shape, _dev(x), cache, 0, router_w=_dev(wr), bias=_dev(b), ws=ws)
    idx_ref, _ = oracle.route(oracle.router_logits(wr, x), b, k)
    assert n == len(np.unique(idx_ref))
    y = coli.layer_fwd(shape, _dev(x), shared_blob=sets[0].shared_blob, router_w=_dev(wr),
                       bias=_dev(b), cache=cache, layer=0, ws=ws)
    yr = coli.layer_fwd(shape, _dev(x), table=sets[0].table, shared_blob=sets[0].shared_blob,
                        router_w=_dev(wr), bias=_dev(b))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), yr.cpu().numpy())
    st = cache.stats()
    assert st["misses"] == 0 and st["prefetch_hits"] == n
    cache.close()


def test_copy_failure_leaves_slot_empty(coli):
    """A copy that cannot be enqueued (forced from the host before any copy is
    issued) returns COLI_EHIP, leaves its slot empty and counts nothing; the
    next lookup of that expert copies it, and the layer output is unchanged."""
    import torch
    L, H, I, E, k, slots = 1, 256, 128, 8, 2, 4
    shape, sets, cache = _setup(coli, L, H, I, E, k, 0, slots)
    try:
        cache.ensure(0, [0, 1, 2, 3])                 # fills the four slots
        cache.wait(0)                                 # (a copied slot counts as late until waited on)
        cache.release(0)
        torch.cuda.synchronize()
        before = cache.stats()
        coli.debug_fail_copies(1)
        with pytest.raises(coli.ColiError) as ei:
            cache.ensure(0, [4])                      # would evict expert 0 (the oldest)
        assert ei.value.code == coli.COLI_EHIP
        after = cache.stats()
        for key in ("misses", "evictions", "bytes_h2d"):
            assert after[key] == before[key], key
        coli.debug_fail_copies(0)
        # expert 4 is not resident and the failed slot's old occupant is gone:
        # both are copied (4 into the empty slot, 0 over the oldest other slot,
        # expert 1's); experts 2 and 3 are still hits
        miss = cache.ensure(0, [4, 0])
        assert miss.tolist() == [1, 1]
        assert cache.stats()["misses"] == before["misses"] + 2
        cache.wait(0)
        cache.release(0)
        miss = cache.ensure(0, [2, 3])
        assert miss.tolist() == [0, 0]
        assert cache.stats()["misses"] == before["misses"] + 2
        cache.wait(0)
        cache.release(0)
        torch.cuda.synchronize()
        # a cached layer call after the failure equals the resident one bit for bit
        x = synth.activations(60, 0, 0, 3, H)
        lg = synth.zipf_logits(60, 0, 0, 3, E, s=1.1)
        coli.debug_fail_copies(0)
        yc = coli.layer_fwd(shape, _dev(x), shared_blob=sets[0].shared_blob, logits=_dev(lg),
                            cache=cache, layer=0)
        yr = coli.layer_fwd(shape, _dev(x), table=sets[0].table, shared_blob=sets[0].shared_blob,
                            logits=_dev(lg))
        torch.cuda.synchronize()
        assert torch.equal(yc, yr)
    finally:
        coli.debug_fail_copies(0)
        cache.close()
