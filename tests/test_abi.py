"""The C-ABI library loads, exports every symbol the header declares, and
rejects bad arguments before touching the GPU (no device needed)."""
import ctypes
import os
import re

import pytest

import int4_routed_expert_sigmoid_amd as coli

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coli_moe.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(coli_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(coli.SO_PATH):
        from int4_routed_expert_sigmoid_amd import build
        build.build()
    return coli.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert "coli_moe_layer_fwd" in names and "coli_expert_cache_ensure" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(coli.EXPORTED) == set(names)


def test_blob_layout_sizes(L):
    off, nbytes = coli.blob_layout(coli.MoEShape(6144, 2048, 256, 1, 8, 0))
    assert nbytes == 18_915_328
    # gate and up rows interleaved in 16-row blocks: up starts 16 rows of 3072 B after gate
    assert off == [0, 49152, 12582912, 18874368, 18882560, 18890752]
    off, nbytes = coli.blob_layout(coli.MoEShape(6144, 2048, 256, 1, 8, 64))
    assert nbytes == 21_233_664
    assert all(o % 256 == 0 for o in off)
    _, tiny = coli.blob_layout(coli.MoEShape(256, 128, 8, 1, 2, 0))
    assert tiny == 51_200


def test_workspace_grows_with_tokens(L):
    s = coli.MoEShape(6144, 2048, 256, 1, 8, 0)
    assert 0 < coli.workspace_size(s, 1) < coli.workspace_size(s, 8) < coli.workspace_size(s, 2048)


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=100), coli.COLI_EINVAL), (dict(group=32), coli.COLI_EUNSUPPORTED),
    (dict(top_k=9, n_routed=8), coli.COLI_EUNSUPPORTED), (dict(n_routed=2000), coli.COLI_EUNSUPPORTED),
    (dict(n_shared=2), coli.COLI_EUNSUPPORTED), (dict(group=64, inter=96), coli.COLI_EINVAL),
    (dict(routed_scale=float("nan")), coli.COLI_EINVAL),
])
def test_shape_validation(L, kw, code):
    base = dict(hidden=256, inter=128, n_routed=8, n_shared=1, top_k=2, group=0, routed_scale=1.0)
    base.update(kw)
    with pytest.raises(coli.ColiError) as ei:
        coli.blob_layout(coli.MoEShape(**base))
    assert ei.value.code == code


def test_argument_errors_before_launch(L):
    vp = ctypes.c_void_p
    assert L.coli_moe_route(vp(1), None, 1, 0, 1, vp(1), vp(1), None) == coli.COLI_EINVAL
    assert L.coli_moe_route(vp(1), None, 1, 8, 9, vp(1), vp(1), None) == coli.COLI_EINVAL
    assert L.coli_moe_route(vp(1), None, 1, 2048, 8, vp(1), vp(1), None) == coli.COLI_EUNSUPPORTED
    assert L.coli_moe_route(None, None, 1, 8, 2, vp(1), vp(1), None) == coli.COLI_EINVAL
    assert b"NULL" in L.coli_last_error()
    assert L.coli_quantize_int4(vp(1), 4, 7, 0, vp(1), vp(1), None) == coli.COLI_EINVAL
    assert L.coli_quantize_int4(vp(1), 4, 96, 64, vp(1), vp(1), None) == coli.COLI_EINVAL
    assert L.coli_quantize_int4(vp(1), 4, 64, 16, vp(1), vp(1), None) == coli.COLI_EUNSUPPORTED
    assert L.coli_moe_union(vp(1), 1, 8, 256, vp(1), vp(1), vp(1), vp(1), vp(1), vp(1), 0,
                            None) == coli.COLI_ENOMEM
    s = coli.MoEShape(256, 128, 8, 1, 2, 0).c()
    # both or neither of logits / router_w
    assert L.coli_moe_layer_fwd(ctypes.byref(s), vp(1), 1, None, None, None, vp(1), vp(1), None, 0,
                                vp(1), None, None, 0, vp(1), 1 << 30, None) == coli.COLI_EINVAL
    assert L.coli_moe_layer_fwd(ctypes.byref(s), vp(1), 1, vp(1), vp(1), None, vp(1), vp(1), None,
                                0, vp(1), None, None, 0, vp(1), 1 << 30, None) == coli.COLI_EINVAL
    # shared blob required with n_shared = 1
    assert L.coli_moe_layer_fwd(ctypes.byref(s), vp(1), 1, vp(1), None, None, vp(1), None, None,
                                0, vp(1), None, None, 0, vp(1), 1 << 30, None) == coli.COLI_EINVAL
    # workspace too small
    assert L.coli_moe_layer_fwd(ctypes.byref(s), vp(1), 1, vp(1), None, None, vp(1), vp(1), None,
                                0, vp(1), None, None, 0, vp(1), 16, None) == coli.COLI_ENOMEM
    assert L.coli_moe_layer_fwd(ctypes.byref(s), vp(1), 1, vp(1), None, None, vp(1), vp(1), None,
                                0, vp(1), None, None, 7, vp(1), 1 << 30, None) == coli.COLI_EINVAL
    # T = 0 is a no-op
    assert L.coli_moe_layer_fwd(ctypes.byref(s), None, 0, vp(1), None, None, vp(1), vp(1), None,
                                0, None, None, None, 0, None, 0, None) == coli.COLI_OK


def test_read_probe_argument_errors(L):
    vp = ctypes.c_void_p
    # NULL buffers, sizes that are not whole 16-byte loads
    assert L.coli_read_probe(None, 1 << 20, 0, 4096, 0, vp(1), 1 << 20, None) == coli.COLI_EINVAL
    assert L.coli_read_probe(vp(1), 1000, 0, 4096, 0, vp(1), 1 << 20, None) == coli.COLI_EINVAL
    # chunk not a multiple of 4096; sink too small for one word per wave
    assert L.coli_read_probe(vp(1), 1 << 20, 0, 3000, 0, vp(1), 1 << 20, None) == coli.COLI_EINVAL
    assert L.coli_read_probe(vp(1), 1 << 20, 0, 4096, 0, vp(1), 16, None) == coli.COLI_EINVAL
    # rows: 48 threads per row neither divide 256 nor make a 3-wave row
    assert L.coli_read_probe(vp(1), 768 * 64, 1, 768, 8, vp(1), 1 << 20, None) == coli.COLI_EINVAL
    # rows: bytes not a whole number of rows; no rows per workgroup; unknown pattern
    assert L.coli_read_probe(vp(1), 3072 * 3 + 16, 1, 3072, 16, vp(1), 1 << 20, None) == coli.COLI_EINVAL
    assert L.coli_read_probe(vp(1), 3072 * 3, 1, 3072, 0, vp(1), 1 << 20, None) == coli.COLI_EINVAL
    assert L.coli_read_probe(vp(1), 1 << 20, 2, 4096, 0, vp(1), 1 << 20, None) == coli.COLI_EINVAL


def test_read_log_argument_errors(L):
    vp = ctypes.c_void_p
    try:
        # negative capacity; a capacity without a records buffer
        assert L.coli_debug_read_log(vp(16), vp(32), -1) == coli.COLI_EINVAL
        assert L.coli_debug_read_log(vp(16), None, 4) == coli.COLI_EINVAL
        # a count with no capacity (counts only) is accepted: this only records the
        # pointers, nothing runs here
        assert L.coli_debug_read_log(vp(16), None, 0) == coli.COLI_OK
    finally:
        # never leave a stand-in address behind for a later launch in this process
        assert L.coli_debug_read_log(None, None, 0) == coli.COLI_OK
