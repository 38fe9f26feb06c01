"""Pins of the oracle's adaptive expert top-p (the practical guide "colibrì 實戰
指南：以純 C 引擎在消費級硬體上串流運行 744B MoE 模型", section 三 and the section 五
tuning table). The pages name the setting but give no formula; the reading
pinned here keeps the shortest key-order prefix of the k selected experts
whose share of their sigmoid scores reaches p, renormalised over the prefix.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth
from tests.numpy_refs import sigmoid_f32

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    logits, cases = None, []
    with open(os.path.join(GOLD, "topp_worked_example.txt")) as f:
        for line in f:
            if line.startswith("logits:"):
                logits = np.array([float(v) for v in line.split(":")[1].split()], np.float32)
            elif line.startswith("case:"):
                p, b2, kept, w = [part.strip() for part in line.split(":", 1)[1].split("|")]
                cases.append((float(p), float(b2), [int(v) for v in kept.split()],
                              [float(v) for v in w.split()]))
    return logits, cases


def test_worked_example():
    logits, cases = _golden()
    k = 4
    for p, b2, kept, wref in cases:
        bias = np.zeros(8, np.float32)
        bias[2] = b2
        idx, w = oracle.route(logits[None, :], bias, k, topp=p)
        n = len(kept)
        assert idx[0, :n].tolist() == kept, (p, b2)
        assert np.all(idx[0, n:] == -1) and np.all(w[0, n:] == 0.0)
        assert np.allclose(w[0, :n], wref, rtol=0, atol=2e-6), (p, b2, w[0])


@pytest.mark.parametrize("p,kept", [(0.1, 1), (0.2, 2), (0.3, 3), (0.5, 4), (0.55, 5), (0.7, 6),
                                    (0.75, 6), (0.85, 7), (0.9, 8), (0.999, 8)])
def test_equal_scores_closed_form(p, kept):
    # equal scores: the share of j+1 slots is (j+1)/k, so ceil(p k) are kept
    # (a share equal to p reaches it: 0.5 and 0.75 sit on a boundary), equal
    # keys go to the lower index, and each kept weight is 1/kept
    k, E = 8, 32
    lg = np.full((3, E), 0.25, np.float32)
    assert kept == math.ceil(p * k)
    idx, w = oracle.route(lg, None, k, topp=p)
    for t in range(3):
        assert idx[t].tolist() == list(range(kept)) + [-1] * (k - kept)
        assert np.all(w[t, :kept] == np.float32(1.0 / kept)) and np.all(w[t, kept:] == 0)


def test_zero_scores_use_slot_count():
    # every score underflows to 0: the weights are uniform, the shares (j+1)/k
    lg = np.full((1, 16), -200.0, np.float32)
    idx, w = oracle.route(lg, None, 4, topp=0.6)
    assert idx[0].tolist() == [0, 1, 2, -1]
    assert np.all(w[0, :3] == np.float32(1.0 / 3))


@pytest.mark.parametrize("p", [0.0, 1.0])
def test_off_values_are_fixed_top_k(p):
    lg = synth.zipf_logits(5, 0, 0, 32, 256, s=1.1)
    b = synth.bias(5, 0, 256)
    i0, w0 = oracle.route(lg, b, 8)
    i1, w1 = oracle.route(lg, b, 8, topp=p)
    assert np.array_equal(i0, i1) and np.array_equal(w0, w1)


def test_prefix_minimal_and_monotone():
    T, E, k = 256, 256, 8
    lg = synth.zipf_logits(6, 0, 0, T, E, s=1.1)
    b = synth.bias(6, 0, E)
    full, _ = oracle.route(lg, b, k)
    s = sigmoid_f32(lg).astype(np.float64)
    sel = np.take_along_axis(s, full.astype(np.int64), axis=1)
    share = np.cumsum(sel, axis=1) / sel.sum(axis=1, keepdims=True)
    prev = np.ones(T, np.int64)
    for p in (0.2, 0.4, 0.6, 0.7, 0.8, 0.95):
        idx, w = oracle.route(lg, b, k, topp=p)
        kept = (idx >= 0).sum(axis=1)
        for t in range(T):
            n = kept[t]
            # a prefix of the fixed top-k, the rest dropped
            assert np.array_equal(idx[t, :n], full[t, :n]) and np.all(idx[t, n:] == -1)
            # minimal: the share reaches p at n slots and not before (away from ties)
            if abs(share[t, n - 1] - p) > 1e-12 and (n < 2 or abs(share[t, n - 2] - p) > 1e-12):
                assert share[t, n - 1] >= p and (n == 1 or share[t, n - 2] < p)
            # renormalised over the kept slots
            ref = sel[t, :n] / sel[t, :n].sum()
            assert np.allclose(w[t, :n], ref, rtol=2e-7, atol=0) and np.all(w[t, n:] == 0)
        assert np.all(kept >= prev)          # more mass asked, never fewer experts
        prev = kept


def test_layer_equals_fixed_top_k_per_token():
    # a token that keeps n slots gets exactly the layer output of top-n routing
    H, I, E, k, T = 128, 64, 16, 4, 6
    experts = [oracle.QExpert.quantize(*synth.expert_weights(7, 0, e, H, I), 0) for e in range(E)]
    shared = oracle.QExpert.quantize(*synth.expert_weights(7, 0, E, H, I), 0)
    lg = synth.zipf_logits(7, 0, 0, T, E, s=1.1)
    x = synth.activations(7, 0, 0, T, H)
    _, y64, idx, w = oracle.layer(x, experts, shared, k, 0, 2.5, logits=lg, topp=0.6)
    kept = (idx >= 0).sum(axis=1)
    assert kept.min() < k                   # the case exercises dropped slots
    for t in range(T):
        n = int(kept[t])
        _, y_n, idx_n, w_n = oracle.layer(x[t:t + 1], experts, shared, n, 0, 2.5,
                                          logits=lg[t:t + 1])
        assert np.array_equal(idx_n[0], idx[t, :n]) and np.array_equal(w_n[0], w[t, :n])
        assert np.array_equal(y_n[0], y64[t])


def test_union_skips_dropped_slots():
    idx = np.array([[3, 1, -1, -1], [1, -1, -1, -1], [0, 3, 2, -1]], np.int32)
    counts, offsets, perm, unique = oracle.union(idx, 5)
    assert counts.tolist() == [1, 2, 1, 2, 0]
    assert offsets.tolist() == [0, 1, 3, 4, 6, 6]
    assert perm[:6].tolist() == [8, 1, 4, 10, 0, 9]
    assert unique.tolist() == [0, 1, 2, 3]


def test_bad_p_rejected():
    lg = np.zeros((1, 8), np.float32)
    for p in (-0.1, 1.5, float("nan")):
        with pytest.raises(ValueError):
            oracle.route(lg, None, 4, topp=p)
