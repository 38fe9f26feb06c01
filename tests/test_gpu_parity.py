"""GPU path vs the CPU oracle, element by element on the same seeded inputs.

Bar: quantiser bytes/scales, routing indices, union arrays bit-exact; routing
weights exact (same double arithmetic); expert/layer outputs max per-row
relative L2 <= 1e-3 on the GEMV path."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import blob_q_rows, ExpertSet, rel_l2_rows

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module")
def coli():
    import torch
    import int4_routed_expert_sigmoid_amd as c
    c.lib()
    assert torch.cuda.is_available()
    return c


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


# ------------------------------------------------------------------ quantiser
@pytest.mark.parametrize("rows,cols,group", [
    (1, 4, 0), (3, 6, 0), (7, 250, 0), (64, 256, 0), (33, 6144, 0), (2048, 2048, 0),
    (5, 64, 64), (17, 192, 64), (129, 6144, 64), (2048, 2048, 64), (0, 64, 0),
])
def test_quantize_bit_exact(coli, rows, cols, group):
    import torch
    w = synth.normal(1, synth.TAG_WEIGHT, rows, cols, rows * cols, 0.0, 0.02).reshape(rows, cols)
    if rows >= 3:
        w[1] = 0.0                                   # all-zero row
        w[2, ::3] *= 100.0                           # a wide row
    q, s = coli.quantize_int4(_dev(w), group)
    torch.cuda.synchronize()
    if rows == 0:
        return
    q_ref, s_ref = oracle.quantize_int4(w, group)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def _near_half_rows(n_rows, seed):
    """Rows of 64 values whose quotients w / scale land on, or within a few ulps
    of, half-integers: element 0 is the row maximum m (so scale = m / 7), the
    others are h * scale for half-integers |h| <= 6.5, nudged by -3..3 ulps.
    Rows with m = 7 (scale 1) and m = 3.5 (scale 0.5) give exact halves; the
    others give quotients just either side of them, where the kernels' fast
    quotient must defer to the exact division."""
    rng = np.random.default_rng(seed)
    halves = np.arange(-6.5, 7.0, 1.0)
    rows = []
    for r in range(n_rows):
        m = np.float32([7.0, 3.5, 1.0, 0.3, 2.0 ** -3, 13.7][r % 6] * (1 + (r // 6) * 0.173))
        scale = np.float32(m / np.float32(7.0))
        h = rng.choice(halves, 63)
        v = (h * np.float64(scale)).astype(np.float32)
        nudge = rng.integers(-3, 4, 63) if r % 6 >= 2 else np.zeros(63, np.int64)
        for step in range(3):                      # |nudge| one-ulp steps toward its sign
            toward = np.where(nudge > 0, np.float32(np.inf), np.float32(-np.inf))
            v = np.where(np.abs(nudge) > step, np.nextafter(v, toward), v).astype(np.float32)
        row = np.concatenate([[m], v]).astype(np.float32)
        rng.shuffle(row)
        rows.append(row)
    return np.stack(rows)


@pytest.mark.parametrize("group", [0, 64])
def test_quantize_near_half_quotients(coli, group):
    import torch
    w = _near_half_rows(96, 5)
    if group == 64:
        w = w.reshape(24, 256)                      # four groups per row, each with its own max
    q, s = coli.quantize_int4(_dev(w), group)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_int4(w, group)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    # the exact halves are really there (scale 1 rows: w itself is the quotient)
    exact = w.reshape(-1, 64)[0]
    assert np.any(np.abs(exact - np.round(exact)) == 0.5)


def test_quantize_expert_layout(coli):
    import torch
    shape = coli.MoEShape(256, 128, 8, 1, 2, 64)
    off, nbytes = coli.blob_layout(shape)
    g, u, d = synth.expert_weights(3, 0, 1, 256, 128)
    blob = coli.quantize_expert(shape, _dev(g), _dev(u), _dev(d)).cpu().numpy()
    qe = oracle.QExpert.quantize(g, u, d, 64)
    parts = qe.parts
    for i, p in enumerate(parts):
        if i < 3:                                    # weight rows (gate and up interleaved)
            raw = blob_q_rows(blob, off, i, p.shape[0], p.shape[1]).reshape(-1)
        else:
            raw = blob[off[i]:off[i] + p.nbytes]
        assert np.array_equal(raw, p.reshape(-1).view(np.uint8)), f"part {i}"


# --------------------------------------------------------------------- router
@pytest.mark.parametrize("T,E,H", [(4, 8, 256), (1, 256, 6144), (33, 64, 512)])
def test_router_logits(coli, T, E, H):
    import torch
    wr = synth.router_weights(2, 0, E, H)
    x = synth.activations(2, 0, 0, T, H)
    lg = coli.router_logits(_dev(wr), _dev(x))
    torch.cuda.synchronize()
    ref = oracle.router_logits(wr, x)
    got = lg.cpu().numpy()
    # double accumulation in another order: equal after the rounding to float
    # except where the double sums straddle a float rounding boundary (1 ulp)
    ulps = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1
    assert (ulps > 0).mean() < 1e-3


@pytest.mark.parametrize("T,E,k,kind", [
    (4, 8, 2, "router"), (1, 256, 8, "router"), (8, 256, 8, "zipf"), (2048, 256, 8, "zipf_mix"),
    (37, 1024, 32, "zipf"), (5, 64, 1, "zipf"), (16, 256, 8, "ties"), (3, 8, 8, "zipf"),
])
def test_route_bit_exact(coli, T, E, k, kind):
    import torch
    if kind == "router":
        H = 256 if E == 8 else 6144
        lg = oracle.router_logits(synth.router_weights(0, 0, E, H), synth.activations(0, 0, 0, T, H))
        b = synth.bias(0, 0, E)
    elif kind == "ties":
        lg = np.round(synth.zipf_logits(9, 0, 0, T, E), 1).astype(np.float32)
        b = np.zeros(E, np.float32)
        b[::7] = 0.125
    else:
        lg = synth.zipf_logits(9, 0, 0, T, E, s=1.1, mix=0.1 if kind == "zipf_mix" else 0.0)
        b = synth.bias(9, 0, E)
    idx, w = coli.route(_dev(lg), _dev(b), k)
    torch.cuda.synchronize()
    idx_ref, w_ref = oracle.route(lg, b, k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert np.array_equal(w.cpu().numpy(), w_ref)


def test_route_no_bias(coli):
    import torch
    lg = synth.zipf_logits(4, 0, 0, 64, 256)
    idx, w = coli.route(_dev(lg), None, 8)
    torch.cuda.synchronize()
    idx_ref, w_ref = oracle.route(lg, None, 8)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert np.array_equal(w.cpu().numpy(), w_ref)


# ---------------------------------------------------------------------- union
@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (8, 8, 256), (4, 2, 8), (2048, 8, 256),
                                   (1000, 3, 1024), (7, 1, 5), (0, 8, 256), (130, 8, 16)])
def test_union_bit_exact(coli, T, k, E):
    import torch
    if T > 0:
        idx_np, _ = oracle.route(synth.zipf_logits(6, 0, 0, T, E, s=1.1), None, k)
    else:
        idx_np = np.zeros((0, k), np.int32)
    idx = _dev(idx_np) if T > 0 else torch.zeros((0, k), dtype=torch.int32, device="cuda")
    counts, offsets, perm, unique, n_unique = coli.union(idx, E)
    torch.cuda.synchronize()
    c, o, p, u = oracle.union(idx_np, E)
    nu = int(n_unique.cpu()[0])
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(perm.cpu().numpy(), p)
    assert nu == len(u) and np.array_equal(unique.cpu().numpy()[:nu], u)


# ----------------------------------------------------------------- expert FFN
@pytest.mark.parametrize("H,I,group,T,k,E", [
    (256, 128, 0, 4, 2, 8), (256, 128, 64, 4, 2, 8), (512, 256, 0, 1, 8, 16),
    (192, 320, 64, 9, 3, 6), (6144, 2048, 0, 1, 8, 256), (6144, 2048, 64, 8, 8, 256),
    (2048, 512, 0, 17, 4, 8),
])
def test_expert_ffn(coli, H, I, group, T, k, E):
    import torch
    shape = coli.MoEShape(H, I, E, 0, k, group)
    lg = synth.zipf_logits(8, 0, 0, T, E, s=1.1)
    idx_np, _ = oracle.route(lg, None, k)
    c, o, p, u = oracle.union(idx_np, E)
    ex = ExpertSet(coli, shape, seed=8, which=u, shared=False)
    x = synth.activations(8, 0, 0, T, H)
    offsets, perm = _dev(o), _dev(p)
    uu = np.zeros(E, np.int32)
    uu[:len(u)] = u
    y = coli.expert_ffn(shape, ex.table, _dev(x), offsets, perm, _dev(uu),
                        _dev(np.array([len(u)], np.int32)), path=coli.PATH_GEMV)
    torch.cuda.synchronize()
    ref = oracle.expert_ffn_union(ex.oracle_list(), x, k, o, p, u, H, I, group)
    err = rel_l2_rows(y.cpu().numpy(), ref)
    assert err.max() <= TOL, f"max rel L2 {err.max():.3e}"


# ---------------------------------------------------------------------- layer
def _layer_case(coli, H, I, E, k, group, T, seed, routing, rs=1.0, n_shared=1, path=None,
                wbits=4):
    import torch
    shape = coli.MoEShape(H, I, E, n_shared, k, group, rs, wbits=wbits)
    x = synth.activations(seed, 0, 0, T, H)
    wr = b = lg = None
    if routing == "router":
        wr = synth.router_weights(seed, 0, E, H)
        b = synth.bias(seed, 0, E)
        lg_sel = oracle.router_logits(wr, x)
    else:
        lg = synth.zipf_logits(seed, 0, 0, T, E, s=1.1, mix=0.1 if routing == "zipf_mix" else 0.0)
        lg_sel = lg
    idx_sel, _ = oracle.route(lg_sel, b, k)
    ex = ExpertSet(coli, shape, seed=seed, which=np.unique(idx_sel), shared=n_shared == 1)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = coli.layer_fwd(shape, _dev(x), table=ex.table, shared_blob=ex.shared_blob,
                       logits=None if lg is None else _dev(lg),
                       router_w=None if wr is None else _dev(wr),
                       bias=None if b is None else _dev(b), idx_out=idx, w_out=w,
                       path=coli.PATH_GEMV if path is None else path)
    torch.cuda.synchronize()
    y_ref, y64, idx_ref, w_ref = oracle.layer(x, ex.oracle_list(), ex.shared_oracle, k, group, rs,
                                              logits=lg, wr=wr, bias=b)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert np.array_equal(w.cpu().numpy(), w_ref)
    err = rel_l2_rows(y.cpu().numpy(), y64)
    tol = 2e-2 if path == coli.PATH_MFMA else TOL          # bf16 activations on the MFMA path
    assert err.max() <= tol, f"max rel L2 {err.max():.3e}"
    return err


@pytest.mark.parametrize("group", [0, 64])
def test_layer_tiny(coli, group):
    _layer_case(coli, 256, 128, 8, 2, group, 4, 0, "router")


def test_layer_decode_glm_shape(coli):
    # decode launch configuration: hidden 6144, inter 2048, 256 + 1 experts, top-8, T = 1,
    # per-row scales, logits from the f32 router; several tokens one call at a time
    for t in range(3):
        _layer_case(coli, 6144, 2048, 256, 8, 0, 1, 100 + t, "router")


def test_layer_mtp_verify_glm_shape(coli):
    # MTP-verify launch configuration: gs64, T = 8, Zipf(1.1) routing
    _layer_case(coli, 6144, 2048, 256, 8, 64, 8, 7, "zipf")


@pytest.mark.parametrize("T,k,group,wbits,path", [
    (1, 2, 0, 4, "gemv"),      # one token: routing folded into gate/up, 8 rows per down wave
    (3, 2, 64, 4, "gemv"),     # a small gs64 batch
    (20, 1, 0, 4, "mfma"),     # the bf16 MFMA path, 256 k steps of gate/up
    (1, 2, 0, 8, "gemv"),      # int8 experts
])
def test_layer_largest_shape(coli, T, k, group, wbits, path):
    # the largest sizes the library accepts: hidden 16384 (8 blocks of 32 columns per
    # lane in gate/up), inter 4096 (2 per lane in down)
    p = coli.PATH_MFMA if path == "mfma" else coli.PATH_GEMV
    _layer_case(coli, 16384, 4096, 4, k, group, T, 21 + T, "router", path=p, wbits=wbits)


def test_layer_routed_scale_no_shared(coli):
    _layer_case(coli, 512, 256, 16, 4, 0, 5, 3, "zipf", rs=2.5, n_shared=0)


@pytest.mark.parametrize("E,k,n_shared,routing,seed", [
    (16, 4, 0, "zipf", 11),        # one token, no shared expert: items start at the first routed one
    (200, 8, 1, "router", 12),     # expert count not a multiple of 64
    (256, 32, 1, "zipf", 13),      # the largest top_k
    (1000, 8, 1, "zipf", 14),      # beyond the folded routing's 256 experts: separate plan pass
    (8, 8, 1, "router", 15),       # k == E
])
def test_layer_one_token_shapes(coli, E, k, n_shared, routing, seed):
    # one-token calls route inside the gate/up pass for E <= 256; the routing
    # published for the later passes and the caller must match the oracle exactly
    for t in range(2):
        _layer_case(coli, 512, 256, E, k, 0, 1, seed * 10 + t, routing, rs=1.5, n_shared=n_shared)


def test_prepared_layer_call_matches_layer_fwd(coli):
    # the prepared-argument call used by decode loops is the same entry point
    import torch
    H, I, E, k = 512, 256, 16, 4
    shape = coli.MoEShape(H, I, E, 1, k, 0)
    ex = ExpertSet(coli, shape, seed=16)
    wr, b = _dev(synth.router_weights(16, 0, E, H)), _dev(synth.bias(16, 0, E))
    x = _dev(synth.activations(16, 0, 0, 3, H))
    ws = coli.workspace(shape, 1)
    call = coli.LayerCall(shape, 1, ws, table=ex.table, shared_blob=ex.shared_blob, router_w=wr,
                          bias=b)
    y = torch.empty((3, H), dtype=torch.float32, device="cuda")
    idx = torch.empty((3, k), dtype=torch.int32, device="cuda")
    for t in range(3):
        call(x.data_ptr() + t * H * 4, y.data_ptr() + t * H * 4, idx.data_ptr() + t * k * 4)
    for t in range(3):
        i1 = torch.empty((1, k), dtype=torch.int32, device="cuda")
        y1 = coli.layer_fwd(shape, x[t:t + 1], table=ex.table, shared_blob=ex.shared_blob,
                            router_w=wr, bias=b, idx_out=i1)
        torch.cuda.synchronize()
        assert torch.equal(y1[0], y[t]) and torch.equal(i1[0], idx[t])
