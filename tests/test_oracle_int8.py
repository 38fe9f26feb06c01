"""Pins of the oracle's int8 codec (the MTP head must be int8: the int8-MTP
page and the practical guide's section 二; rule read as the int4 container
rule of the model card with 127 in place of 7)."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.numpy_refs import dequant8, ffn_dense, quantize8_numpy

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example():
    d = {}
    with open(os.path.join(GOLD, "int8_worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            d[k.strip()] = [float(x) for x in v.split()]
    q, s = oracle.quantize_int8(np.array([d["w"]], np.float32))
    assert s.tolist() == d["scale"]
    assert q[0].tolist() == [int(v) for v in d["q"]]


@pytest.mark.parametrize("rows,cols,group", [(64, 256, 0), (33, 192, 64), (5, 6, 0)])
def test_matches_numpy_rint(rows, cols, group):
    w = synth.expert_matrix(21, 0, 1, 0, rows, cols)
    q, s = oracle.quantize_int8(w, group)
    q2, s2 = quantize8_numpy(w, group)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    # every value within half a step, the largest magnitude at +-127
    step = s.reshape(rows, -1).repeat(cols if group == 0 else 64, axis=1)
    assert np.all(np.abs(q.astype(np.float64) * step - w) <= step / 2 * (1 + 1e-6))
    assert np.all(np.abs(q).max(axis=1) == 127)


def test_zero_rows_and_extremes():
    w = np.zeros((2, 64), np.float32)
    w[1, 3] = -5.0
    q, s = oracle.quantize_int8(w)
    assert s[0] == 0 and np.all(q[0] == 0)
    assert q[1, 3] == -127 and np.count_nonzero(q[1]) == 1


@pytest.mark.parametrize("H,I,group", [(256, 128, 0), (128, 192, 64)])
def test_int8_ffn_matches_dense_numpy(H, I, group):
    g, u, d = synth.expert_weights(22, 0, 0, H, I)
    ex = oracle.QExpert.quantize(g, u, d, group, bits=8)
    x = synth.activations(22, 0, 0, 3, H)
    y = oracle.expert_ffn(ex, x, H, I, group)
    gq, uq, dq, gs, us, ds = ex.parts
    ref = ffn_dense(dequant8(gq, gs, group), dequant8(uq, us, group), dequant8(dq, ds, group), x)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    # int8 is closer to the f32 weights than int4
    ref32 = ffn_dense(g.astype(np.float64), u.astype(np.float64), d.astype(np.float64), x)
    y4 = oracle.expert_ffn(oracle.QExpert.quantize(g, u, d, group), x, H, I, group)
    assert np.linalg.norm(y - ref32) < np.linalg.norm(y4 - ref32) / 4


def test_int8_layer_mixes_with_int4_shared():
    # a layer may hold int8 routed experts; the combine is unchanged
    H, I, E, k, T = 128, 64, 6, 2, 3
    ex8 = [oracle.QExpert.quantize(*synth.expert_weights(23, 0, e, H, I), 0, bits=8) for e in range(E)]
    sh8 = oracle.QExpert.quantize(*synth.expert_weights(23, 0, E, H, I), 0, bits=8)
    lg = synth.zipf_logits(23, 0, 0, T, E)
    x = synth.activations(23, 0, 0, T, H)
    _, y64, idx, w = oracle.layer(x, ex8, sh8, k, 0, 1.0, logits=lg)
    for t in range(T):
        ref = oracle.expert_ffn(sh8, x[t], H, I, 0)[0]
        for j in range(k):
            ref = ref + float(w[t, j]) * oracle.expert_ffn(ex8[idx[t, j]], x[t], H, I, 0)[0]
        assert np.allclose(y64[t], ref, rtol=1e-12, atol=1e-15)
