"""Pins of the oracle's sigmoid router (DeepSeek-V3-style sigmoid scores, a
selection-only bias, top-k of 256, normalised weights: the lbrq.cn article's
section 三 item 1 and section 四 item 3; scoring_func sigmoid and
norm_topk_prob from the config.json values quoted by the int8-MTP page)."""
import numpy as np
import pytest

import oracle
import synth
from tests.numpy_refs import best_subset, route_by_rank, sigmoid_f32


def test_rank_definition_glm_shape():
    lg = synth.zipf_logits(0, 0, 0, 64, 256, s=1.1)
    b = synth.bias(0, 0, 256)
    idx, w = oracle.route(lg, b, 8)
    idx2, s = route_by_rank(lg, b, 8)
    assert np.array_equal(idx, idx2)
    # weights: unbiased scores normalised over the selected, sums ~1
    sel = np.take_along_axis(s.astype(np.float64), idx.astype(np.int64), axis=1)
    ref = (sel / sel.cumsum(axis=1)[:, -1:]).astype(np.float32)   # slot-order sum
    assert np.array_equal(w, ref)
    assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1.0) <= 1e-6)
    assert all(len(set(r)) == 8 for r in idx.tolist())


def test_bias_changes_selection_not_weights():
    lg = synth.zipf_logits(1, 0, 0, 16, 256, s=1.1)
    b = np.zeros(256, np.float32)
    b[5] = 10.0                       # expert 5 always selected first
    idx, w = oracle.route(lg, b, 8)
    assert np.all(idx[:, 0] == 5)
    s = sigmoid_f32(lg)
    sel = np.take_along_axis(s.astype(np.float64), idx.astype(np.int64), axis=1)
    assert np.array_equal(w, (sel / sel.cumsum(axis=1)[:, -1:]).astype(np.float32))


def test_tiny_config_exhaustive():
    H, E, k, T = 256, 8, 2, 4
    wr = synth.router_weights(0, 0, E, H)
    x = synth.activations(0, 0, 0, T, H)
    b = synth.bias(0, 0, E)
    lg = oracle.router_logits(wr, x)
    idx, _ = oracle.route(lg, b, k)
    s = sigmoid_f32(lg)
    key = (s + b[None, :]).astype(np.float32)
    for t in range(T):
        assert sorted(idx[t].tolist()) == list(best_subset(key[t], k))
        assert key[t, idx[t, 0]] >= key[t, idx[t, 1]]


def test_zero_bias_is_stable_argsort():
    lg = synth.normal(4, synth.TAG_GUMBEL, 0, 0, 32 * 256, 0.0, 1.57).reshape(32, 256)
    idx, _ = oracle.route(lg, None, 8)
    s = sigmoid_f32(lg)
    ref = np.argsort(-s, axis=1, kind="stable")[:, :8]
    assert np.array_equal(idx, ref)
    # where the float32 scores are all distinct the order is the logit order
    for t in range(32):
        if len(np.unique(s[t])) == 256:
            assert np.array_equal(idx[t], np.argsort(-lg[t], kind="stable")[:8])


def test_ties_go_to_lower_index():
    lg = np.zeros((2, 16), np.float32)
    lg[1, [3, 9, 12]] = 1.0
    idx, w = oracle.route(lg, None, 4)
    assert idx[0].tolist() == [0, 1, 2, 3]
    assert idx[1].tolist() == [3, 9, 12, 0]
    assert np.all(w[0] == np.float32(0.25))


def test_zero_score_sum():
    # sigmoid of -200 rounds to 0 in float32: the weights fall back to 1/k
    lg = np.full((1, 8), -200.0, np.float32)
    idx, w = oracle.route(lg, None, 4)
    assert idx[0].tolist() == [0, 1, 2, 3]
    assert np.all(w == np.float32(0.25))


def test_router_logits_numpy():
    wr = synth.router_weights(2, 0, 64, 512)
    x = synth.activations(2, 0, 0, 5, 512)
    lg = oracle.router_logits(wr, x)
    ref = (x.astype(np.float64) @ wr.astype(np.float64).T)
    assert np.max(np.abs(lg - ref) / np.abs(ref).max()) < 1e-7
    assert np.array_equal(lg, ref.astype(np.float32)) or np.max(np.abs(lg - ref.astype(np.float32))) <= \
        np.spacing(np.abs(ref).astype(np.float32)).max()


def test_bad_arguments():
    with pytest.raises(ValueError):
        oracle.route(np.zeros((1, 4), np.float32), None, 5)
