"""coli_moe_layer_fwd_noalloc (the layer on the library's static device
scratch, for callers that cannot allocate) against coli_moe_layer_fwd with a
workspace: two calls in a row on each launch path, the second with fewer
tokens, must give the same routing and bit-identical outputs (same kernels),
and both meet the oracle's bar; a call too large for the scratch is refused
before anything is enqueued."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import ExpertSet, rel_l2_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def coli():
    import int4_routed_expert_sigmoid_amd as c
    c.lib()
    return c


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _pair(coli, shape, ex, x, wr=None, b=None, lg=None, path=0):
    """(workspace call, no-alloc call) outputs: y, idx, w of each."""
    import torch
    T, k = x.shape[0], shape.top_k
    outs = []
    for fn in ("ws", "noalloc"):
        y = torch.full((T, shape.hidden), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
        w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
        kw = dict(table=ex.table, shared_blob=ex.shared_blob,
                  logits=None if lg is None else _dev(lg), router_w=None if wr is None else _dev(wr),
                  bias=None if b is None else _dev(b), y=y, idx_out=idx, w_out=w, path=path)
        if fn == "ws":
            coli.layer_fwd(shape, _dev(x), **kw)
        else:
            coli.layer_fwd_noalloc(shape, _dev(x), **kw)
        outs.append((y, idx, w))
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("group,path,T1,T2,topp", [
    (0, "gemv", 8, 1, 0.0),        # small-batch GEMV, then one token (routing folded into gate/up)
    (64, "gemv", 12, 3, 0.0),      # gs64 batches
    (0, "mfma", 40, 20, 0.0),      # bf16 MFMA grouped GEMM
    (0, "auto", 33, 2, 0.0),       # auto: MFMA, then the GEMV family
    (0, "gemv", 6, 1, 0.6),        # adaptive expert top-p
])
def test_noalloc_matches_layer_fwd(coli, group, path, T1, T2, topp):
    import torch
    H, I, E, k, seed = 512, 256, 16, 4, 71
    shape = coli.MoEShape(H, I, E, 1, k, group, 1.0, topp)
    ex = ExpertSet(coli, shape, seed=seed)
    wr, b = synth.router_weights(seed, 0, E, H), synth.bias(seed, 0, E)
    p = {"gemv": coli.PATH_GEMV, "mfma": coli.PATH_MFMA, "auto": coli.PATH_AUTO}[path]
    first = 0
    for T in (T1, T2):                            # two calls in a row, the second smaller
        x = synth.activations(seed, 0, first, T, H)
        first += T
        (y_ws, i_ws, w_ws), (y_na, i_na, w_na) = _pair(coli, shape, ex, x, wr=wr, b=b, path=p)
        assert torch.equal(i_na, i_ws) and torch.equal(w_na, w_ws)
        assert torch.equal(y_na, y_ws)
        _, y64, idx_ref, w_ref = oracle.layer(x, ex.oracle_list(), ex.shared_oracle, k, group, 1.0,
                                              wr=wr, bias=b, topp=topp)
        assert np.array_equal(i_na.cpu().numpy(), idx_ref)
        assert np.array_equal(w_na.cpu().numpy(), w_ref)
        tol = 2e-2 if (p == coli.PATH_MFMA or (p == coli.PATH_AUTO and T > 16)) else 1e-3
        err = rel_l2_rows(y_na.cpu().numpy(), y64)
        assert err.max() <= tol, f"T={T}: max rel L2 {err.max():.3e}"


def test_noalloc_glm_decode_shape(coli):
    """Hidden 6144, inter 2048, 256 + 1 experts, top-8: an 8-token batch, then
    one token (the decode launch sequence)."""
    import torch
    H, I, E, k, seed = 6144, 2048, 256, 8, 72
    shape = coli.MoEShape(H, I, E, 1, k, 0)
    wr, b = synth.router_weights(seed, 0, E, H), synth.bias(seed, 0, E)
    xs = [synth.activations(seed, 0, 0, 8, H), synth.activations(seed, 0, 8, 1, H)]
    need = np.unique(np.concatenate([oracle.route(oracle.router_logits(wr, x), b, k)[0].ravel()
                                     for x in xs]))
    ex = ExpertSet(coli, shape, seed=seed, which=need)
    for x in xs:
        (y_ws, i_ws, w_ws), (y_na, i_na, w_na) = _pair(coli, shape, ex, x, wr=wr, b=b,
                                                       path=coli.PATH_GEMV)
        assert torch.equal(i_na, i_ws) and torch.equal(w_na, w_ws) and torch.equal(y_na, y_ws)
        _, y64, idx_ref, _ = oracle.layer(x, ex.oracle_list(), ex.shared_oracle, k, 0, 1.0,
                                          wr=wr, bias=b)
        assert np.array_equal(i_na.cpu().numpy(), idx_ref)
        assert rel_l2_rows(y_na.cpu().numpy(), y64).max() <= 1e-3


def test_noalloc_refuses_calls_beyond_the_scratch(coli):
    import torch
    H, I, E, k = 6144, 2048, 256, 8
    shape = coli.MoEShape(H, I, E, 1, k, 0)
    T = 400                                        # workspace about 131 MB, above the 64 MiB scratch
    assert coli.workspace_size(shape, T) > 64 << 20
    x = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    lg = torch.zeros((T, E), dtype=torch.float32, device="cuda")
    table = torch.zeros(E, dtype=torch.int64, device="cuda")
    shared = torch.zeros(16, dtype=torch.uint8, device="cuda")
    y = torch.full((T, H), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(coli.ColiError) as ei:
        coli.layer_fwd_noalloc(shape, x, table, shared_blob=shared, logits=lg, y=y)
    assert ei.value.code == coli.COLI_ENOMEM and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())                  # nothing was enqueued
