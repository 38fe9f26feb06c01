"""The seeded input generator: Philox4x32-10 known answers, determinism, ranges."""
import os

import numpy as np

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    n = 0
    for line in open(os.path.join(GOLD, "philox4x32_10_kat.txt")):
        if line.startswith("#") or not line.strip():
            continue
        v = [int(t, 16) for t in line.split()]
        out = synth.philox4x32_10(v[0:4], v[4:6])
        assert list(out) == v[6:10]
        n += 1
    assert n == 3


def test_normal_is_counter_based():
    a = synth.normal(0, synth.TAG_WEIGHT, 3, 5, 10001, 0.0, 0.02)
    b = synth.normal(0, synth.TAG_WEIGHT, 3, 5, 777, 0.0, 0.02, first=4321)
    assert np.array_equal(a[4321:4321 + 777], b)
    c = synth.normal(0, synth.TAG_WEIGHT, 3, 6, 10001, 0.0, 0.02)
    assert not np.array_equal(a, c)
    assert np.array_equal(a, synth.normal(0, synth.TAG_WEIGHT, 3, 5, 10001, 0.0, 0.02))


def test_normal_moments():
    a = synth.normal(1, synth.TAG_X, 0, 0, 2_000_000).astype(np.float64)
    assert abs(a.mean()) < 3e-3
    assert abs(a.std() - 1.0) < 3e-3
    # fourth moment of a normal is 3
    assert abs(np.mean(a ** 4) - 3.0) < 0.05


def test_permutation_and_zipf():
    p = synth.popularity_perm(0, 0, 256)
    assert sorted(p.tolist()) == list(range(256))
    lg = synth.zipf_logits(0, 0, 0, 4000, 256, s=1.1)
    top1 = lg.argmax(axis=1)
    # the most popular expert (rank 0) is the most frequent top-1 pick
    counts = np.bincount(top1, minlength=256)
    assert counts.argmax() == int(np.where(p == 0)[0][0])


def test_locality_logits_encode_chosen_sets():
    lg, chosen = synth.locality_logits(0, 2, 64, 256, 8, keep_p=0.6)
    for t in range(64):
        top = set(np.argsort(-lg[t])[:8].tolist())
        assert top == set(chosen[t].tolist())
        assert len(top) == 8
    kept = [len(set(chosen[t]) & set(chosen[t - 1])) for t in range(1, 64)]
    assert 3.0 < np.mean(kept) < 7.0
