"""Pins of the oracle's FP8 -> f32 -> int4 converter (model card
"jlnsrk/GLM-5.2-colibri-int4", conversion note: FP8 e4m3 with one scale per
128 x 128 block, to f32, to int4 with np.rint)."""
import math
import os

import numpy as np
import pytest

import oracle
import synth
from tests.numpy_refs import quantize_numpy

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_values_from_the_format():
    n = 0
    with open(os.path.join(GOLD, "fp8_e4m3_values.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code, val = line.split()
            got = oracle.fp8_e4m3_value(int(code, 16))
            if val == "nan":
                assert math.isnan(got)
            else:
                assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))
            n += 1
    assert n == 17


def test_e4m3_all_codes_match_torch():
    import torch
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.fp8_e4m3_value(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("rows,cols", [(128, 128), (300, 200), (1, 130), (257, 64)])
def test_block_dequant_indexing(rows, cols):
    rng = np.random.default_rng(rows * 1000 + cols)
    codes = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                  # no NaN codes
    br, bc = (rows + 127) // 128, (cols + 127) // 128
    scale = np.exp2(rng.integers(-12, 4, size=(br, bc))).astype(np.float32) * \
        rng.uniform(0.5, 1.0, size=(br, bc)).astype(np.float32)
    import torch
    val = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    full = np.repeat(np.repeat(scale.astype(np.float64), 128, 0), 128, 1)[:rows, :cols]
    ref = (val * full).astype(np.float32)                 # exact product, one rounding
    got = oracle.fp8_block_dequant(codes, scale)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("group", [0, 64])
def test_converter_is_dequant_then_quantise(group):
    codes, scale = synth.fp8_block_matrix(3, 0, 1, synth.MAT_GATE, 256, 384)
    q, s = oracle.convert_fp8_int4(codes, scale, group)
    w = oracle.fp8_block_dequant(codes, scale)
    q2, s2, _ = quantize_numpy(w, group)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_converted_weights_track_the_original():
    # end to end: f32 -> FP8 (block scaled) -> f32 -> int4 stays within the two
    # rounding steps of the original weights
    rows, cols = 256, 512
    w = synth.expert_matrix(4, 0, 2, synth.MAT_UP, rows, cols)
    codes, scale = synth.fp8_block_matrix(4, 0, 2, synth.MAT_UP, rows, cols)
    q, s = oracle.convert_fp8_int4(codes, scale, 64)
    deq = oracle.dequantize_int4(q, s, cols, 64)
    step = np.repeat(s, 64, axis=1)
    w8 = oracle.fp8_block_dequant(codes, scale).astype(np.float64)
    assert np.all(np.abs(w8 - w) <= np.abs(w) * 2.0 ** -4 + 2.0 ** -9 * scale.max())
    assert np.all(np.abs(deq - w8) <= step / 2 * (1 + 1e-6))
