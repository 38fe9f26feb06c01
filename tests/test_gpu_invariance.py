"""Properties of the GEMV path that hold at any size.

- Batch invariance: a token's layer output does not depend on the batch it
  is computed in (the draft/verify lesson of the practical guide, section 二:
  both must compute the same function). Per token, the integer block sums are
  exact and the float reductions run in the same order for any batch, so the
  outputs must be bit-identical.
- Reuse: the same workspace serves consecutive calls without being cleared
  (every call writes each region it reads), and repeated calls give identical
  bits.
"""
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


@pytest.fixture(scope="module")
def layer_setup(coli):
    H, I, E, k, T = 2048, 512, 64, 8, 17
    shape = coli.MoEShape(H, I, E, 1, k, 0, 1.0)
    ex = ExpertSet(coli, shape, seed=21)
    x = synth.activations(21, 0, 0, T, H)
    lg = synth.zipf_logits(21, 0, 0, T, E, s=1.1)
    b = synth.bias(21, 0, E)
    return shape, ex, x, lg, b


@pytest.mark.parametrize("batch", [8, 17])
def test_batch_invariance(coli, layer_setup, batch):
    import torch
    shape, ex, x, lg, b = layer_setup
    ws = coli.workspace(shape, 17, coli.PATH_GEMV)
    singles = []
    for t in range(batch):
        y = coli.layer_fwd(shape, _dev(x[t:t + 1]), table=ex.table, shared_blob=ex.shared_blob,
                           logits=_dev(lg[t:t + 1]), bias=_dev(b), path=coli.PATH_GEMV, ws=ws)
        singles.append(y)
    yb = coli.layer_fwd(shape, _dev(x[:batch]), table=ex.table, shared_blob=ex.shared_blob,
                        logits=_dev(lg[:batch]), bias=_dev(b), path=coli.PATH_GEMV, ws=ws)
    torch.cuda.synchronize()
    ys = torch.cat(singles).cpu().numpy()
    assert np.array_equal(yb.cpu().numpy(), ys)
    _, y64, _, _ = oracle.layer(x[:batch], ex.oracle_list(), ex.shared_oracle, shape.top_k, 0, 1.0,
                                logits=lg[:batch], bias=b)
    assert rel_l2_rows(ys, y64).max() <= 1e-3


def test_workspace_reuse_and_repeatability(coli, layer_setup):
    import torch
    shape, ex, x, lg, b = layer_setup
    ws = coli.workspace(shape, 8, coli.PATH_GEMV)
    outs = []
    for _ in range(3):
        y = coli.layer_fwd(shape, _dev(x[:8]), table=ex.table, shared_blob=ex.shared_blob,
                           logits=_dev(lg[:8]), bias=_dev(b), path=coli.PATH_GEMV, ws=ws)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    # the workspace is reused without clearing: every call writes what it reads
    _, y64, _, _ = oracle.layer(x[:8], ex.oracle_list(), ex.shared_oracle, shape.top_k, 0, 1.0,
                                logits=lg[:8], bias=b)
    assert rel_l2_rows(outs[2], y64).max() <= 1e-3


@pytest.mark.parametrize("H,I,E,k,group,shared,topp,rs,wbits", [
    (6144, 2048, 256, 8, 0, True, 0.0, 1.0, 4),     # the GLM layer
    (1120, 2048, 64, 9, 0, True, 0.0, 0.7, 4),      # 10 work items, routed scale
    (512, 256, 16, 1, 64, False, 0.0, 2.5, 4),      # gs64, no shared expert, k = 1
    (768, 512, 32, 8, 0, True, 0.7, 1.0, 4),        # top-p: dropped slots
    (768, 512, 300, 4, 0, True, 0.0, 1.0, 4),       # E > 256: routing not folded
    (32, 64, 8, 2, 0, True, 0.0, 1.0, 4),           # two blocks per row
    (512, 4096, 16, 4, 0, True, 0.0, 1.0, 4),       # inter 4096
    (512, 256, 16, 4, 0, True, 0.0, 1.0, 8),        # int8 experts
    (256, 2048, 16, 15, 0, True, 0.0, 1.0, 4),      # 16 work items
])
def test_one_token_equals_its_row_in_a_batch(coli, H, I, E, k, group, shared, topp, rs, wbits):
    """A one-token call (routing folded into the gate/up pass, its own launch
    bodies) gives the same bits as that token's row of a 3-token call."""
    import torch
    shape = coli.MoEShape(H, I, E, 1 if shared else 0, k, group, rs, topp, wbits)
    T = 3
    x = synth.activations(23, 0, 0, T, H)
    lg = synth.zipf_logits(23, 0, 0, T, E, s=1.1)
    b = synth.bias(23, 0, E)
    used = np.unique(oracle.route(lg, b, k, topp=topp)[0])
    ex = ExpertSet(coli, shape, seed=23, which=used[used >= 0], shared=shared, keep_oracle=set())
    sb = ex.shared_blob if shared else None
    ws = coli.workspace(shape, T, coli.PATH_GEMV)
    singles = []
    for t in range(T):
        y = coli.layer_fwd(shape, _dev(x[t:t + 1]), table=ex.table, shared_blob=sb,
                           logits=_dev(lg[t:t + 1]), bias=_dev(b), path=coli.PATH_GEMV, ws=ws)
        singles.append(y)
    yb = coli.layer_fwd(shape, _dev(x), table=ex.table, shared_blob=sb, logits=_dev(lg),
                        bias=_dev(b), path=coli.PATH_GEMV, ws=ws)
    torch.cuda.synchronize()
    ys = torch.cat(singles).cpu().numpy()
    assert np.isfinite(ys).all()
    assert np.array_equal(yb.cpu().numpy(), ys)
