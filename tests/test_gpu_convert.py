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


def _offset_view(a, off, dtype):
    """A contiguous device view of array a that starts `off` elements into a
    larger buffer (off = 0: an ordinary aligned tensor)."""
    import torch
    a = np.ascontiguousarray(a)
    buf = torch.zeros(a.size + off, dtype=dtype, device="cuda")
    buf[off:].copy_(torch.from_numpy(a.reshape(-1)))
    return buf[off:].view(a.shape)


@pytest.mark.parametrize("group", [0, 64])
@pytest.mark.parametrize("offs", [(1, 0, 0), (8, 8, 3), (0, 1, 16)])
def test_expert_blob_from_unaligned_matrices(coli, group, offs):
    """Gate and up are converted together when both take the wave path; a
    gate or up matrix that starts off a 16-byte boundary sends the pair to
    separate launches (one of them the byte-wise path). Every blob part still
    equals the oracle's conversion bit for bit."""
    import torch
    H, I = 256, 128
    shape = coli.MoEShape(H, I, 8, 1, 2, group)
    dims = ((I, H), (I, H), (H, I))
    mats = [synth.fp8_block_matrix(10, 0, 12, m, r, c)
            for m, (r, c) in zip((synth.MAT_GATE, synth.MAT_UP, synth.MAT_DOWN), dims)]
    args = []
    for (codes, scale), o in zip(mats, offs):
        args += [_offset_view(codes, o, torch.uint8), _dev(scale)]
    blob = coli.convert_fp8_expert(shape, *args)
    torch.cuda.synchronize()
    off, _ = coli.blob_layout(shape)
    b = blob.cpu().numpy()
    for i, ((codes, scale), (r, c)) in enumerate(zip(mats, dims)):
        q_ref, s_ref = oracle.convert_fp8_int4(codes, scale, group)
        q = blob_q_rows(b, off, i, r, q_ref.shape[1]).reshape(q_ref.shape)
        s = b[off[3 + i]:off[3 + i] + s_ref.nbytes].view(np.float32).reshape(s_ref.shape)
        assert np.array_equal(q, q_ref), i
        assert np.array_equal(s, s_ref), i


@pytest.mark.parametrize("group", [0, 64])
@pytest.mark.parametrize("offs", [(1, 0, 0), (0, 3, 1), (1, 1, 0), (1, 1, 1)])
def test_quantize_expert_unaligned_matrices(coli, group, offs):
    """f32 expert matrices off a 16-byte boundary. Per-row scales: the three
    matrices share one launch only when all three are aligned alike (all
    unaligned: element-wise loads and byte stores); otherwise gate and up go
    through the pair launch (itself split when only one of them is unaligned)
    and down through its own. Bit-exact against the oracle's quantizer."""
    import torch
    H, I = 256, 128
    shape = coli.MoEShape(H, I, 8, 1, 2, group)
    g, u, d = synth.expert_weights(4, 0, 1, H, I)
    views = [_offset_view(a, o, torch.float32) for a, o in zip((g, u, d), offs)]
    blob = coli.quantize_expert(shape, *views).cpu().numpy()
    qe = oracle.QExpert.quantize(g, u, d, group)
    off, _ = coli.blob_layout(shape)
    for i, p in enumerate(qe.parts):
        if i < 3:
            raw = blob_q_rows(blob, off, i, p.shape[0], p.shape[1]).reshape(-1)
        else:
            raw = blob[off[i]:off[i] + p.nbytes]
        assert np.array_equal(raw, p.reshape(-1).view(np.uint8)), f"part {i}"
