"""Pins of the oracle's batch union (the lbrq.cn article's section 三 item 4 and
the practical guide's section 二: positions hitting the same expert are merged
so each unique expert is read once)."""
import numpy as np
import pytest

import oracle
import synth
from tests.numpy_refs import union_numpy


@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (8, 8, 256), (4, 2, 8), (2048, 8, 256), (3, 1, 5)])
def test_union_matches_sort_and_count(T, k, E):
    lg = synth.zipf_logits(5, 1, 0, T, E, s=1.1)
    idx, _ = oracle.route(lg, None, k)
    counts, offsets, perm, unique = oracle.union(idx, E)
    c2, o2, p2, u2 = union_numpy(idx, E)
    assert np.array_equal(counts, c2)
    assert np.array_equal(offsets, o2)
    assert np.array_equal(perm, p2)
    assert np.array_equal(unique, u2)
    # invariants
    assert counts.sum() == T * k and offsets[-1] == T * k
    assert sorted(perm.tolist()) == list(range(T * k))
    flat = idx.reshape(-1)
    for e in unique:
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(flat[seg] == e)


def test_identical_tokens():
    idx = np.tile(np.array([[7, 3, 9]], np.int32), (5, 1))
    counts, offsets, perm, unique = oracle.union(idx, 12)
    assert unique.tolist() == [3, 7, 9]
    assert counts[3] == counts[7] == counts[9] == 5
    assert perm[offsets[3]:offsets[4]].tolist() == [1, 4, 7, 10, 13]


def test_empty_batch():
    counts, offsets, perm, unique = oracle.union(np.zeros((0, 8), np.int32), 256)
    assert counts.sum() == 0 and offsets[-1] == 0 and len(perm) == 0 and len(unique) == 0


def test_out_of_range_rejected():
    with pytest.raises(ValueError):
        oracle.union(np.array([[0, 9]], np.int32), 8)
