"""Seeded random layer shapes through coli_moe_layer_fwd against the oracle.

Each case draws its own shape and options:
- hidden and inter sizes (multiples of 64, including ones that are not multiples
  of the kernels' tiles);
- the routed expert count, top-k and token count;
- per-row or gs64 scales, with or without a shared expert, and a routed scale;
- routing from f32 router weights with a bias, or from given logits;
- adaptive expert top-p, int4 or int8 experts, and the FFN path.

Every case checks routing and weights bit for bit and the output within the
path's tolerance. The cases are fixed by their seeds, so a failure names its
shape and reproduces."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import ExpertSet, rel_l2_rows

pytestmark = pytest.mark.gpu

N_CASES = 64


@pytest.fixture(scope="module")
def coli():
    import int4_routed_expert_sigmoid_amd as c
    c.lib()
    return c


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _draw(seed):
    r = np.random.default_rng(1000 + seed)
    H = int(r.choice([64, 128, 192, 256, 384, 512, 1024]))
    I = int(r.choice([64, 128, 192, 320, 512]))
    E = int(r.choice([4, 8, 13, 16, 64, 200, 256, 300]))
    k = int(min(E, r.choice([1, 2, 4, 8])))
    T = int(r.choice([1, 1, 2, 5, 8, 17, 33, 70]))
    group = int(r.choice([0, 64]))
    n_shared = int(r.choice([0, 1]))
    rs = float(r.choice([1.0, 2.5]))
    routing = str(r.choice(["router", "logits"]))
    topp = float(r.choice([0.0, 0.0, 0.6]))
    wbits = int(r.choice([4, 4, 8]))
    path = str(r.choice(["auto", "gemv", "mfma"]))
    if wbits == 8:
        path = "gemv"                       # the MFMA path is int4 only
    return dict(H=H, I=I, E=E, k=k, T=T, group=group, n_shared=n_shared, rs=rs,
                routing=routing, topp=topp, wbits=wbits, path=path)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_layer_shapes(coli, seed):
    import torch
    c = _draw(seed)
    H, I, E, k, T, group = c["H"], c["I"], c["E"], c["k"], c["T"], c["group"]
    shape = coli.MoEShape(H, I, E, c["n_shared"], k, group, c["rs"], topp=c["topp"],
                          wbits=c["wbits"])
    x = synth.activations(seed, 0, 0, T, H)
    wr = b = lg = None
    if c["routing"] == "router":
        wr = synth.router_weights(seed, 0, E, H)
        b = synth.bias(seed, 0, E)
        lg_sel = oracle.router_logits(wr, x)
    else:
        lg = synth.zipf_logits(seed, 0, 0, T, E, s=1.1, mix=0.1)
        lg_sel = lg
    idx_sel, _ = oracle.route(lg_sel, b, k)
    ex = ExpertSet(coli, shape, seed=seed, which=np.unique(idx_sel), shared=c["n_shared"] == 1)
    path = {"auto": coli.PATH_AUTO, "gemv": coli.PATH_GEMV, "mfma": coli.PATH_MFMA}[c["path"]]
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = coli.layer_fwd(shape, _dev(x), table=ex.table, shared_blob=ex.shared_blob,
                       logits=None if lg is None else _dev(lg),
                       router_w=None if wr is None else _dev(wr),
                       bias=None if b is None else _dev(b), idx_out=idx, w_out=w, path=path)
    torch.cuda.synchronize()
    _, y64, idx_ref, w_ref = oracle.layer(x, ex.oracle_list(), ex.shared_oracle, k, group, c["rs"],
                                          logits=lg, wr=wr, bias=b, topp=c["topp"])
    assert np.array_equal(idx.cpu().numpy(), idx_ref), f"case {c}: routing"
    assert np.array_equal(w.cpu().numpy(), w_ref), f"case {c}: weights"
    # bf16 activations on the MFMA path (auto takes it for T > 16 with int4)
    mfma = c["path"] == "mfma" or (c["path"] == "auto" and T > 16 and c["wbits"] == 4)
    tol = 2e-2 if mfma else 1e-3
    err = rel_l2_rows(y.cpu().numpy(), y64)
    assert err.max() <= tol, f"case {c}: max rel L2 {err.max():.3e}"
