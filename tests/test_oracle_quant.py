"""Pins of the oracle's int4 quantiser (container rule of the model card
"jlnsrk/GLM-5.2-colibri-int4": packed nibbles + F32 scales, np.rint rounding;
gs64 from the practical guide's section 三)."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.numpy_refs import quantize_numpy, unpack_nibbles

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_example():
    d = {}
    for line in open(os.path.join(GOLD, "quant_worked_example.txt")):
        if line.startswith("#") or ":" not in line:
            continue
        key, val = line.split(":", 1)
        d[key.strip()] = val.split()
    return d


def test_worked_example_half_even():
    d = _golden_example()
    w = np.array([[float(v) for v in d["w"]]], dtype=np.float32)
    q, s = oracle.quantize_int4(w, 0)
    assert s[0] == np.float32(float(d["scale"][0]))
    assert [int(b) for b in q[0]] == [int(b, 16) for b in d["bytes"]]
    assert unpack_nibbles(q, 4)[0].tolist() == [int(v) for v in d["q"]]


@pytest.mark.parametrize("group", [0, 64])
def test_matches_numpy_rint(group):
    rng_w = synth.normal(7, synth.TAG_WEIGHT, 0, 0, 4096 * 256, 0.0, 0.02).reshape(4096, 256)
    # add exact halves so that ties are exercised: w = (n + 0.5) * scale
    w = rng_w.copy()
    w[:64, 1] = np.float32(3.5) * (np.abs(w[:64]).max(axis=1) / np.float32(7))
    q, s = oracle.quantize_int4(w, group)
    q2, s2, _ = quantize_numpy(w, group)
    assert np.array_equal(s, s2)
    assert np.array_equal(q, q2)


@pytest.mark.parametrize("group", [0, 64])
def test_invariants(group):
    w = synth.normal(3, synth.TAG_WEIGHT, 1, 1, 512 * 384, 0.0, 0.02).reshape(512, 384)
    q, s = oracle.quantize_int4(w, group)
    v = unpack_nibbles(q, 384).astype(np.float64)
    span = 384 if group == 0 else 64
    sc = np.repeat(np.asarray(s, np.float64).reshape(512, -1), span, axis=1)
    err = np.abs(w.astype(np.float64) - v * sc)
    assert np.all(err <= sc / 2 * (1 + 1e-6) + 1e-30)
    # the largest |w| of every row/group maps to +-7
    wg = np.abs(w).reshape(512, -1, span)
    am = wg.argmax(axis=2)
    vg = v.reshape(512, -1, span)
    picked = np.take_along_axis(vg, am[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.abs(picked) == 7)
    assert v.min() >= -8 and v.max() <= 7
    # the oracle's own dequantiser agrees with the numpy unpacking
    deq = oracle.dequantize_int4(q, s, 384, group)
    assert np.array_equal(deq, v * sc)


def test_zero_rows_and_groups():
    w = np.zeros((3, 128), np.float32)
    w[1, 70] = -0.5
    q, s = oracle.quantize_int4(w, 64)
    assert s[0].tolist() == [0.0, 0.0]
    assert s[1, 0] == 0.0 and s[1, 1] == np.float32(0.5) / np.float32(7)
    assert np.all(q[0] == 0) and np.all(q[2] == 0)
    v = unpack_nibbles(q, 128)
    assert v[1, 70] == -7 and np.count_nonzero(v) == 1


def test_minus_eight_decodes():
    # the quantiser never emits -8 (|w|/scale <= 7) but the format holds it
    q = np.array([[0x88]], np.uint8)
    assert unpack_nibbles(q, 2).tolist() == [[-8, -8]]
    assert oracle.dequantize_int4(q, np.array([0.5], np.float32), 2, 0).tolist() == [[-4.0, -4.0]]


def test_bad_arguments():
    with pytest.raises(ValueError):
        oracle.quantize_int4(np.zeros((2, 3), np.float32), 0)
    with pytest.raises(ValueError):
        oracle.quantize_int4(np.zeros((2, 96), np.float32), 64)
