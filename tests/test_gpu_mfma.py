"""bf16-MFMA grouped GEMM path vs the CPU oracle.

Bar: max per-row relative L2 error <= 2e-2 (bf16 activations, f32
accumulation); routing and union stay bit-exact (same kernels as the GEMV
path)."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import ExpertSet, rel_l2_rows

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def coli():
    import int4_routed_expert_sigmoid_amd as c
    c.lib()
    return c


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


@pytest.mark.parametrize("H,I,group,T,k,E", [
    (256, 128, 0, 4, 2, 8), (256, 128, 64, 4, 2, 8), (512, 256, 0, 1, 8, 16),
    (192, 320, 64, 9, 3, 6), (1024, 512, 0, 100, 4, 8), (512, 384, 64, 130, 6, 12),
    # experts with 128-token tiles and remainders of every size; a half-live
    # last row block (I = 320) and fewer k steps than one unrolled group (H = 192)
    (512, 256, 0, 300, 4, 8), (192, 320, 0, 700, 3, 6),
])
def test_expert_ffn_mfma(coli, H, I, group, T, k, E):
    import torch
    shape = coli.MoEShape(H, I, E, 0, k, group)
    lg = synth.zipf_logits(31, 0, 0, T, E, s=1.1)
    idx_np, _ = oracle.route(lg, None, k)
    c, o, p, u = oracle.union(idx_np, E)
    ex = ExpertSet(coli, shape, seed=31, which=u, shared=False)
    x = synth.activations(31, 0, 0, T, H)
    uu = np.zeros(E, np.int32)
    uu[:len(u)] = u
    y = coli.expert_ffn(shape, ex.table, _dev(x), _dev(o), _dev(p), _dev(uu),
                        _dev(np.array([len(u)], np.int32)), path=coli.PATH_MFMA)
    torch.cuda.synchronize()
    ref = oracle.expert_ffn_union(ex.oracle_list(), x, k, o, p, u, H, I, group)
    err = rel_l2_rows(y.cpu().numpy(), ref)
    assert err.max() <= TOL, f"max rel L2 {err.max():.3e}"


@pytest.mark.parametrize("group,T", [(0, 40), (64, 40), (0, 257)])
def test_layer_mfma_small_shapes(coli, group, T):
    import torch
    H, I, E, k = 512, 256, 16, 4
    shape = coli.MoEShape(H, I, E, 1, k, group)
    ex = ExpertSet(coli, shape, seed=33)
    x = synth.activations(33, 0, 0, T, H)
    lg = synth.zipf_logits(33, 0, 0, T, E, s=1.1, mix=0.1)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    y = coli.layer_fwd(shape, _dev(x), table=ex.table, shared_blob=ex.shared_blob,
                       logits=_dev(lg), idx_out=idx, path=coli.PATH_AUTO)
    torch.cuda.synchronize()
    _, y64, idx_ref, _ = oracle.layer(x, ex.oracle_list(), ex.shared_oracle, k, group, 1.0,
                                      logits=lg)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    err = rel_l2_rows(y.cpu().numpy(), y64)
    assert err.max() <= TOL, f"max rel L2 {err.max():.3e}"


def test_layer_prefill_glm_shape_sampled(coli):
    """Prefill launch configuration: hidden 6144, inter 2048, 256 + 1 experts,
    top-8, T = 2048 tokens, per-row scales, Zipf(1.1) + 10% uniform routing.
    Routing and union are checked on every token, the outputs of 12 tokens
    spread over the batch against the oracle."""
    import torch
    H, I, E, k, T = 6144, 2048, 256, 8, 2048
    shape = coli.MoEShape(H, I, E, 1, k, 0)
    lg = synth.zipf_logits(0, 0, 0, T, E, s=1.1, mix=0.1)
    x = synth.activations(0, 0, 0, T, H)
    sample = np.linspace(0, T - 1, 12).astype(int)
    idx_all, _ = oracle.route(lg, None, k)
    need = np.unique(idx_all[sample])
    # all experts are needed on the device; only the sampled tokens' on the host
    ex = ExpertSet(coli, shape, seed=0, which=range(E), keep_oracle=set(need.tolist()))
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    y = coli.layer_fwd(shape, _dev(x), table=ex.table, shared_blob=ex.shared_blob,
                       logits=_dev(lg), idx_out=idx, path=coli.PATH_MFMA)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), idx_all)
    _, y64, _, _ = oracle.layer(x[sample], ex.oracle_list(), ex.shared_oracle, k, 0, 1.0,
                                logits=lg[sample])
    err = rel_l2_rows(y.cpu().numpy()[sample], y64)
    assert err.max() <= TOL, f"max rel L2 {err.max():.3e}"


def test_auto_path_sends_few_token_experts_to_gemv(coli):
    """With the path chosen automatically for a batch above 16 tokens, experts
    with at most 4 tokens run on the GEMV family (f32-accurate, 1e-3) and the
    rest on the bf16 MFMA tiles (2e-2): routing is built so that experts 0-2
    get 2, 4 and 5 tokens and experts 3-7 the rest."""
    import torch
    H, I, E, k, T = 512, 256, 8, 2, 40
    shape = coli.MoEShape(H, I, E, 0, k, 0)
    first = [0] * 2 + [1] * 4 + [2] * 5 + [3 + t % 5 for t in range(T - 11)]
    lg = np.full((T, E), -4.0, np.float32)
    for t in range(T):
        lg[t, first[t]] = 4.0
        lg[t, 3 + (t + 2) % 5 if first[t] < 3 else 3 + (first[t] - 3 + 1) % 5] = 3.0
    idx_np, _ = oracle.route(lg, None, k)
    c, o, p, u = oracle.union(idx_np, E)
    assert c[:3].tolist() == [2, 4, 5] and c[3:].min() > 4
    ex = ExpertSet(coli, shape, seed=35, which=u, shared=False)
    x = synth.activations(35, 0, 0, T, H)
    uu = np.zeros(E, np.int32)
    uu[:len(u)] = u
    args = (shape, ex.table, _dev(x), _dev(o), _dev(p), _dev(uu), _dev(np.array([len(u)], np.int32)))
    y_auto = coli.expert_ffn(*args, path=coli.PATH_AUTO)
    y_mfma = coli.expert_ffn(*args, path=coli.PATH_MFMA)
    torch.cuda.synchronize()
    ref = oracle.expert_ffn_union(ex.oracle_list(), x, k, o, p, u, H, I, 0)
    e_auto = rel_l2_rows(y_auto.cpu().numpy(), ref)
    e_mfma = rel_l2_rows(y_mfma.cpu().numpy(), ref)
    expert_of_row = idx_np.reshape(-1)
    small = c[expert_of_row] <= 4
    assert small.sum() == 6
    assert e_auto[small].max() <= 1e-3            # GEMV family
    assert e_auto[~small].max() <= TOL            # MFMA tiles
    assert e_mfma[small].max() > 1e-3             # the same rows on bf16 tiles
    assert np.array_equal(y_auto.cpu().numpy()[~small], y_mfma.cpu().numpy()[~small])
