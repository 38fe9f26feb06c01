"""HIP-graph replay of layer calls (how the decode benchmark deploys them)
against the same calls launched eagerly.

The kernels are deterministic, so every replay must reproduce the eager
outputs bit for bit. The graph is replayed several times with the program's
own eager work (other calls through the same workspace) and synchronisations
between the replays, so that state a replay leaves behind, or finds left by
eager work, cannot hide. One case per launch sequence: the one-token call with
the routing folded into the gate/up pass, the small-batch GEMV path (gs64),
and the bf16 MFMA path."""
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


@pytest.mark.parametrize("T,group,path", [(1, 0, "gemv"), (8, 64, "gemv"), (40, 0, "mfma")])
def test_graph_replay_matches_eager(coli, T, group, path):
    import torch
    H, I, E, k, n_calls, seed = 512, 256, 16, 4, 4, 41
    shape = coli.MoEShape(H, I, E, 1, k, group)
    ex = ExpertSet(coli, shape, seed=seed)
    wr, b = synth.router_weights(seed, 0, E, H), synth.bias(seed, 0, E)
    wr_d, b_d = _dev(wr), _dev(b)
    p = coli.PATH_MFMA if path == "mfma" else coli.PATH_GEMV
    x = _dev(synth.activations(seed, 0, 0, n_calls * T, H))
    other = _dev(synth.activations(seed, 0, 1000, T, H))      # eager work between replays
    stream = torch.cuda.Stream()
    ws = coli.workspace(shape, T, p)
    call = coli.LayerCall(shape, T, ws, table=ex.table, shared_blob=ex.shared_blob,
                          router_w=wr_d, bias=b_d, path=p, stream=stream)

    def run(y, idx, xs=x, n=n_calls):
        for c in range(n):
            call(xs.data_ptr() + c * T * H * 4, y.data_ptr() + c * T * H * 4,
                 idx.data_ptr() + c * T * k * 4)

    y_e = torch.empty((n_calls * T, H), dtype=torch.float32, device="cuda")
    i_e = torch.empty((n_calls * T, k), dtype=torch.int32, device="cuda")
    with torch.cuda.stream(stream):
        run(y_e, i_e)
    torch.cuda.synchronize()

    y_g = torch.empty_like(y_e)
    i_g = torch.empty_like(i_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        run(y_g, i_g)
    torch.cuda.synchronize()
    y_o = torch.empty((T, H), dtype=torch.float32, device="cuda")
    i_o = torch.empty((T, k), dtype=torch.int32, device="cuda")
    for rep in range(3):
        y_g.fill_(float("nan"))
        i_g.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(i_g, i_e), f"replay {rep}: routing differs from the eager calls"
        assert torch.equal(y_g, y_e), f"replay {rep}: outputs differ from the eager calls"
        with torch.cuda.stream(stream):                      # eager work on the same workspace
            run(y_o, i_o, xs=other, n=1)
        torch.cuda.synchronize()

    # and the eager outputs are the layer's (first call against the oracle)
    tol = 2e-2 if path == "mfma" else 1e-3
    x0 = synth.activations(seed, 0, 0, T, H)
    _, y64, idx_ref, _ = oracle.layer(x0, ex.oracle_list(), ex.shared_oracle, k, group, 1.0,
                                      wr=wr, bias=b)
    assert np.array_equal(i_e[:T].cpu().numpy(), idx_ref)
    err = rel_l2_rows(y_e[:T].cpu().numpy(), y64)
    assert err.max() <= tol, f"max rel L2 {err.max():.3e}"


@pytest.mark.parametrize("T,group,topp", [(1, 0, 0.0), (8, 64, 0.0), (1, 0, 0.6), (5, 0, 0.6)])
def test_profile_rerun_recomputes_the_call(coli, T, group, topp):
    """coli_profile_rerun (the benchmark's graph of back-to-back GEMV launches)
    enqueues a pass of the last layer call again: the workspace it rewrites
    must come out byte for byte as the call left it, and a graph of reruns
    over several workspaces must leave each one unchanged too."""
    import torch
    H, I, E, k, seed = 512, 256, 16, 4, 43
    shape = coli.MoEShape(H, I, E, 1, k, group, 1.0, topp)
    ex = ExpertSet(coli, shape, seed=seed)
    wr_d, b_d = _dev(synth.router_weights(seed, 0, E, H)), _dev(synth.bias(seed, 0, E))
    n = 3
    x = _dev(synth.activations(seed, 0, 0, n * T, H))
    nb = coli.workspace_size(shape, T, coli.PATH_GEMV)
    ws = torch.empty((n, nb), dtype=torch.uint8, device="cuda")
    for i in range(n):
        coli.layer_fwd(shape, x[i * T:(i + 1) * T], table=ex.table, shared_blob=ex.shared_blob,
                       router_w=wr_d, bias=b_d, path=coli.PATH_GEMV, ws=ws[i])
    torch.cuda.synchronize()
    before = ws.clone()
    for which in (0, 1):
        coli.profile_rerun(shape, T, ex.table, ex.shared_blob, which, ws[0])
    torch.cuda.synchronize()
    assert torch.equal(ws, before)
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(n):
            for which in (0, 1):
                coli.profile_rerun(shape, T, ex.table, ex.shared_blob, which, ws[i], stream=stream)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ws, before)
    with pytest.raises(coli.ColiError):
        coli.profile_rerun(shape, 17, ex.table, ex.shared_blob, 0, ws[0])
