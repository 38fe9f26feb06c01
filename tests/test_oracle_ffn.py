"""Pins of the oracle's expert FFN and layer (SwiGLU gate/up/down stored
adjacently, practical guide section 二; shared expert always applied;
combine by normalised weights with the routed-scale factor)."""
import numpy as np
import pytest

import oracle
import synth
from tests.numpy_refs import dequant, ffn_dense, route_by_rank, union_numpy


def _experts(seed, n, H, I, group, layer=0):
    out = []
    for e in range(n):
        g, u, d = synth.expert_weights(seed, layer, e, H, I)
        out.append(oracle.QExpert.quantize(g, u, d, group))
    return out


def _dense(ex, H, I, group):
    gq, uq, dq, gs, us, ds = ex.parts
    return dequant(gq, gs, H, group), dequant(uq, us, H, group), dequant(dq, ds, I, group)


@pytest.mark.parametrize("H,I,group", [(256, 128, 0), (128, 192, 64), (64, 64, 0), (192, 128, 64)])
def test_ffn_matches_dense_numpy(H, I, group):
    ex = _experts(11, 1, H, I, group)[0]
    x = synth.activations(11, 0, 0, 3, H)
    y = oracle.expert_ffn(ex, x, H, I, group)
    g, u, d = _dense(ex, H, I, group)
    ref = ffn_dense(g, u, d, x)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_ffn_one_hot_input():
    H, I = 128, 64
    ex = _experts(12, 1, H, I, 0)[0]
    g, u, d = _dense(ex, H, I, 0)
    c = 37
    x = np.zeros((1, H), np.float32)
    x[0, c] = 1.0
    y = oracle.expert_ffn(ex, x, H, I, 0)[0]
    gc, uc = g[:, c], u[:, c]                   # column c of the dequantised matrices
    h = gc / (1 + np.exp(-gc)) * uc
    assert np.allclose(y, d @ h, rtol=1e-13, atol=0)


def test_ffn_zero_up_gives_zero():
    H, I = 128, 64
    gate, up, down = synth.expert_weights(13, 0, 0, H, I)
    ex = oracle.QExpert.quantize(gate, np.zeros_like(up), down, 0)
    y = oracle.expert_ffn(ex, synth.activations(13, 0, 0, 2, H), H, I, 0)
    assert np.all(y == 0.0)


def _layer_numpy(x, experts, shared, k, group, rs, logits, bias, H, I):
    idx, s = route_by_rank(logits, bias, k)
    sel = np.take_along_axis(s.astype(np.float64), idx.astype(np.int64), axis=1)
    w = (sel / sel.cumsum(axis=1)[:, -1:]).astype(np.float32)
    dense = [_dense(e, H, I, group) for e in experts]
    y = ffn_dense(*_dense(shared, H, I, group), x) if shared is not None else np.zeros(x.shape)
    for t in range(x.shape[0]):
        acc = np.zeros(H)
        for j in range(k):
            acc += float(w[t, j]) * ffn_dense(*dense[idx[t, j]], x[t:t + 1])[0]
        y[t] += rs * acc
    return y, idx, w


@pytest.mark.parametrize("group", [0, 64])
def test_tiny_layer_matches_numpy(group):
    H, I, E, k, T = 256, 128, 8, 2, 4
    experts = _experts(0, E, H, I, group)
    g, u, d = synth.expert_weights(0, 0, E, H, I)
    shared = oracle.QExpert.quantize(g, u, d, group)
    wr = synth.router_weights(0, 0, E, H)
    b = synth.bias(0, 0, E)
    x = synth.activations(0, 0, 0, T, H)
    y, y64, idx, w = oracle.layer(x, experts, shared, k, group, 1.0, wr=wr, bias=b)
    lg = oracle.router_logits(wr, x)
    ref, idx2, w2 = _layer_numpy(x, experts, shared, k, group, 1.0, lg, b, H, I)
    assert np.array_equal(idx, idx2) and np.array_equal(w, w2)
    assert np.max(np.abs(y64 - ref)) <= 1e-12 * np.max(np.abs(ref))
    assert np.array_equal(y, y64.astype(np.float32))


def test_layer_routed_scale_and_special_cases():
    H, I, E, k, T = 128, 64, 6, 3, 5
    experts = _experts(3, E, H, I, 0)
    g, u, d = synth.expert_weights(3, 0, E, H, I)
    shared = oracle.QExpert.quantize(g, u, d, 0)
    lg = synth.zipf_logits(3, 0, 0, T, E)
    x = synth.activations(3, 0, 0, T, H)
    _, y_sh, _, _ = oracle.layer(x, experts, shared, k, 0, 0.0, logits=lg)
    assert np.allclose(y_sh, oracle.expert_ffn(shared, x, H, I, 0), rtol=0, atol=0)
    _, y1, _, _ = oracle.layer(x, experts, shared, k, 0, 1.0, logits=lg)
    _, y25, _, _ = oracle.layer(x, experts, shared, k, 0, 2.5, logits=lg)
    assert np.allclose(y25 - y_sh, 2.5 * (y1 - y_sh), rtol=1e-12, atol=1e-15)
    # k = 1: the weight is exactly 1 and the output is shared + that expert
    _, y_k1, idx1, w1 = oracle.layer(x, experts, None, 1, 0, 1.0, logits=lg)
    assert np.all(w1 == 1.0)
    for t in range(T):
        assert np.array_equal(y_k1[t], oracle.expert_ffn(experts[idx1[t, 0]], x[t], H, I, 0)[0])
    # identical tokens give identical rows
    xs = np.tile(x[:1], (4, 1))
    ls = np.tile(lg[:1], (4, 1))
    _, yi, idxi, _ = oracle.layer(xs, experts, shared, k, 0, 1.0, logits=ls)
    assert np.all(yi == yi[0]) and np.all(idxi == idxi[0])


def test_ffn_union_segments():
    H, I, E, k, T = 64, 64, 5, 2, 6
    experts = _experts(4, E, H, I, 0)
    lg = synth.zipf_logits(4, 0, 0, T, E)
    idx, _ = oracle.route(lg, None, k)
    counts, offsets, perm, unique = union_numpy(idx, E)
    x = synth.activations(4, 0, 0, T, H)
    ya = oracle.expert_ffn_union(experts, x, k, offsets, perm, unique, H, I, 0)
    for a in range(T * k):
        ref = oracle.expert_ffn(experts[idx.reshape(-1)[a]], x[a // k], H, I, 0)[0]
        assert np.array_equal(ya[a], ref)
