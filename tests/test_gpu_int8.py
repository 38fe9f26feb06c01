"""int8 expert codec on the GPU vs the CPU oracle (the MTP head must be int8:
the int8-MTP page and the practical guide's section 二). The quantiser is
bit-exact (the blob's nibble planes reassemble the oracle's int8 values);
layer outputs meet the GEMV bar (1e-3 relative L2 per row)."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import blob_q_rows, ExpertSet, rel_l2_rows

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module")
def coli():
    import int4_routed_expert_sigmoid_amd as c
    c.lib()
    return c


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _int8_from_planes(part: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Blob part of an int8 matrix -> q int8 [rows][cols]: per 32-column block,
    16 bytes of high nibbles h then 16 bytes of low nibbles l, q = 16 h + l + 8."""
    b = part.reshape(rows, cols // 32, 2, 16)

    def nib(x):
        lo = (x & 15).astype(np.int16)
        hi = (x >> 4).astype(np.int16)
        out = np.empty(x.shape[:-1] + (32,), np.int16)
        out[..., 0::2] = lo
        out[..., 1::2] = hi
        return (out ^ 8) - 8
    q = 16 * nib(b[:, :, 0]) + nib(b[:, :, 1]) + 8
    return q.reshape(rows, cols).astype(np.int8)


@pytest.mark.parametrize("H,I,group", [(256, 128, 0), (512, 320, 64), (6144, 2048, 0)])
def test_int8_blob_bit_exact(coli, H, I, group):
    import torch
    shape = coli.MoEShape(H, I, 8, 1, 2, group, 1.0, 0.0, 8)
    g, u, d = synth.expert_weights(30, 0, 1, H, I)
    blob = coli.quantize_expert(shape, _dev(g), _dev(u), _dev(d))
    torch.cuda.synchronize()
    off, nbytes = coli.blob_layout(shape)
    b = blob.cpu().numpy()
    for i, (w, r, c) in enumerate(((g, I, H), (u, I, H), (d, H, I))):
        q_ref, s_ref = oracle.quantize_int8(w, group)
        q = _int8_from_planes(blob_q_rows(b, off, i, r, c).reshape(-1), r, c)
        s = b[off[3 + i]:off[3 + i] + s_ref.nbytes].view(np.float32).reshape(s_ref.shape)
        assert np.array_equal(q, q_ref), i
        assert np.array_equal(s, s_ref), i


def test_int8_fp8_conversion(coli):
    import torch
    H, I = 512, 256
    shape = coli.MoEShape(H, I, 8, 1, 2, 64, 1.0, 0.0, 8)
    mats = [synth.fp8_block_matrix(31, 0, 2, m, r, c)
            for m, (r, c) in ((synth.MAT_GATE, (I, H)), (synth.MAT_UP, (I, H)), (synth.MAT_DOWN, (H, I)))]
    blob = coli.convert_fp8_expert(shape, *[_dev(a) for pair in mats for a in pair])
    torch.cuda.synchronize()
    off, _ = coli.blob_layout(shape)
    b = blob.cpu().numpy()
    for i, ((codes, scale), (r, c)) in enumerate(zip(mats, ((I, H), (I, H), (H, I)))):
        q_ref, s_ref = oracle.quantize_int8(oracle.fp8_block_dequant(codes, scale), 64)
        assert np.array_equal(_int8_from_planes(blob_q_rows(b, off, i, r, c).reshape(-1), r, c), q_ref), i
        s = b[off[3 + i]:off[3 + i] + s_ref.nbytes].view(np.float32).reshape(s_ref.shape)
        assert np.array_equal(s, s_ref), i


@pytest.mark.parametrize("H,I,E,k,group,T,routing", [
    (6144, 2048, 256, 8, 0, 1, "router"),      # decode shape, int8 experts
    (6144, 2048, 256, 8, 64, 8, "zipf"),       # MTP-verify batch shape, gs64
    (512, 256, 16, 4, 0, 5, "zipf"),
    (512, 320, 16, 4, 64, 40, "zipf"),         # route / union / plan kernels, GEMV for T > 16
    (256, 128, 8, 2, 0, 4, "router"),
])
def test_int8_layer(coli, H, I, E, k, group, T, routing):
    import torch
    shape = coli.MoEShape(H, I, E, 1, k, group, 1.0, 0.0, 8)
    x = synth.activations(32, 0, 0, T, H)
    wr = b = lg = None
    if routing == "router":
        wr = synth.router_weights(32, 0, E, H)
        b = synth.bias(32, 0, E)
        lg_sel = oracle.router_logits(wr, x)
    else:
        lg = synth.zipf_logits(32, 0, 0, T, E, s=1.1, mix=0.1)
        lg_sel = lg
    idx_sel, _ = oracle.route(lg_sel, b, k)
    ex = ExpertSet(coli, shape, seed=32, which=np.unique(idx_sel))
    y = coli.layer_fwd(shape, _dev(x), table=ex.table, shared_blob=ex.shared_blob,
                       logits=None if lg is None else _dev(lg),
                       router_w=None if wr is None else _dev(wr),
                       bias=None if b is None else _dev(b), path=coli.PATH_AUTO)
    torch.cuda.synchronize()
    _, y64, _, _ = oracle.layer(x, ex.oracle_list(), ex.shared_oracle, k, group, 1.0,
                                logits=lg, wr=wr, bias=b)
    err = rel_l2_rows(y.cpu().numpy(), y64)
    assert err.max() <= TOL, f"max rel L2 {err.max():.3e}"


def test_int8_mfma_path_refused(coli):
    shape = coli.MoEShape(512, 256, 16, 1, 4, 0, 1.0, 0.0, 8)
    ex = ExpertSet(coli, shape, seed=33, which=[0])
    x = _dev(synth.activations(33, 0, 0, 40, 512))
    lg = _dev(synth.zipf_logits(33, 0, 0, 40, 16))
    with pytest.raises(coli.ColiError) as ei:
        coli.layer_fwd(shape, x, table=ex.table, shared_blob=ex.shared_blob, logits=lg,
                       path=coli.PATH_MFMA)
    assert ei.value.code == coli.COLI_EUNSUPPORTED
