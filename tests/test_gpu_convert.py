"""FP8 -> f32 -> int4 converter on the GPU vs the CPU oracle (model card
"jlnsrk/GLM-5.2-colibri-int4", conversion note). Integer and byte outputs:
the bar is bit-exact packed nibbles and scales."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import blob_q_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def coli():
    import int4_routed_expert_sigmoid_amd as c
    c.lib()
    return c


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def test_every_code_through_the_row_scale(coli):
    # row r holds one non-NaN code and zeros: its scale is |value| / 7, so the
    # scales pin the decode of all 254 codes
    import torch
    codes = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    w8 = np.zeros((len(codes), 64), np.uint8)
    w8[:, 5] = codes
    scale = np.ones((2, 1), np.float32)
    q, s = coli.convert_fp8_int4(_dev(w8), _dev(scale), 0)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.convert_fp8_int4(w8, scale, 0)
    assert np.array_equal(s.cpu().numpy(), s_ref) and np.array_equal(q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("rows,cols,group", [(300, 200, 0), (257, 384, 64), (1, 130, 0),
                                             (128, 4096, 64), (5, 6, 0)])
def test_random_codes_bit_exact(coli, rows, cols, group):
    import torch
    rng = np.random.default_rng(rows + cols)
    w8 = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    w8[(w8 & 0x7F) == 0x7F] = 0x3F
    br, bc = (rows + 127) // 128, (cols + 127) // 128
    scale = (np.exp2(rng.integers(-14, 2, size=(br, bc))) *
             rng.uniform(0.5, 1.0, size=(br, bc))).astype(np.float32)
    q, s = coli.convert_fp8_int4(_dev(w8), _dev(scale), group)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.convert_fp8_int4(w8, scale, group)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref)


def test_unaligned_views(coli):
    # views that start one byte / one float into their buffers take the
    # byte-wise load and store paths
    import torch
    rows, cols = 40, 256
    codes, scale = synth.fp8_block_matrix(8, 0, 3, synth.MAT_DOWN, rows, cols)
    buf = torch.zeros(rows * cols + 1, dtype=torch.uint8, device="cuda")
    buf[1:].copy_(torch.from_numpy(codes.reshape(-1)))
    w8 = buf[1:].view(rows, cols)
    qbuf = torch.zeros(rows * cols // 2 + 1, dtype=torch.uint8, device="cuda")
    q = qbuf[1:].view(rows, cols // 2)
    q, s = coli.convert_fp8_int4(w8, _dev(scale), 0, q=q)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.convert_fp8_int4(codes, scale, 0)
    assert np.array_equal(q.cpu().numpy(), q_ref) and np.array_equal(s.cpu().numpy(), s_ref)


@pytest.mark.parametrize("group", [0, 64])
def test_glm_expert_blob(coli, group):
    """One GLM-5.2-shaped expert (hidden 6144, inter 2048) from checkpoint-style
    FP8 matrices into a blob; every part equals the oracle's conversion."""
    import torch
    H, I = 6144, 2048
    shape = coli.MoEShape(H, I, 256, 1, 8, group)
    mats = [synth.fp8_block_matrix(9, 0, 11, m, r, c)
            for m, (r, c) in ((synth.MAT_GATE, (I, H)), (synth.MAT_UP, (I, H)),
                              (synth.MAT_DOWN, (H, I)))]
    blob = coli.convert_fp8_expert(shape, *[_dev(a) for pair in mats for a in pair])
    torch.cuda.synchronize()
    off, nbytes = coli.blob_layout(shape)
    b = blob.cpu().numpy()
    for i, ((codes, scale), (r, c)) in enumerate(zip(mats, ((I, H), (I, H), (H, I)))):
        q_ref, s_ref = oracle.convert_fp8_int4(codes, scale, group)
        q = blob_q_rows(b, off, i, r, q_ref.shape[1]).reshape(q_ref.shape)
        s = b[off[3 + i]:off[3 + i] + s_ref.nbytes].view(np.float32).reshape(s_ref.shape)
        assert np.array_equal(q, q_ref), i
        assert np.array_equal(s, s_ref), i
