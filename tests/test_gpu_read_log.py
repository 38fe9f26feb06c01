"""The batch union reads each unique expert's weights once (lbrq.cn article
"github一周涨11k⭐️！25GB 内存跑 744B GLM-5.2 模型！", section 三 item 4;
practical guide section 二).

With the GEMV read log on (coli_debug_read_log), every workgroup that streams
a tile of an expert's weight rows records (blob, pass, tile). The oracle's
routing of the same inputs decides which experts must appear: every expert of
the union, and the shared one, has each gate/up tile and each down tile
streamed once per work item, and no other expert appears (the experts outside
the union all point at one zero blob, so a read of any of them shows as that
blob). One token: one item per expert. Small batches: an expert that c of the
tokens selected is ceil(c / 4) items of consecutive tokens, whose workgroups
for one tile run side by side (so that the rows cross HBM once; the MTP
counter profile checks the bytes), each walking its rows once."""
from collections import Counter

import numpy as np
import pytest

import oracle
import synth
from tests.helpers import ExpertSet

pytestmark = pytest.mark.gpu


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


def _logged_layer(coli, shape, T, seed, routing, topp=0.0, cap=1 << 16):
    """Run one layer call with the read log on; returns (records [n][4] uint32,
    count, oracle idx, ExpertSet)."""
    import torch
    H, E, k = shape.hidden, shape.n_routed, shape.top_k
    x = synth.activations(seed, 0, 0, T, H)
    wr = b = lg = None
    if routing == "router":
        wr = synth.router_weights(seed, 0, E, H)
        b = synth.bias(seed, 0, E)
        lg_sel = oracle.router_logits(wr, x)
    else:
        lg = synth.zipf_logits(seed, 0, 0, T, E, s=1.1)
        lg_sel = lg
    idx_ref, _ = oracle.route(lg_sel, b, k, topp=topp)
    union = np.unique(idx_ref[idx_ref >= 0])
    ex = ExpertSet(coli, shape, seed=seed, which=union, shared=shape.n_shared == 1)
    count = torch.zeros(1, dtype=torch.int32, device="cuda")
    rec = torch.zeros((cap, 4), dtype=torch.int32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    coli.debug_read_log(count, rec)
    try:
        coli.layer_fwd(shape, _dev(x), table=ex.table, shared_blob=ex.shared_blob,
                       logits=None if lg is None else _dev(lg),
                       router_w=None if wr is None else _dev(wr),
                       bias=None if b is None else _dev(b), idx_out=idx, path=coli.PATH_GEMV)
        torch.cuda.synchronize()
    finally:
        coli.debug_read_log()
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    n = int(count.item())
    r = rec[:min(n, cap)].cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    return r, n, idx_ref, ex


def _check_union_read_once(shape, T, recs, idx_ref, ex):
    H, I = shape.hidden, shape.inter
    blob = recs[:, 0] | (recs[:, 1] << 32)
    pas, tile = recs[:, 2] >> 16, recs[:, 2] & 0xFFFF
    rows, walks = recs[:, 3] & 0xFFFF, recs[:, 3] >> 16
    union = np.unique(idx_ref[idx_ref >= 0])
    expect = {int(ex.blobs[e].data_ptr()): int((idx_ref == e).sum()) for e in union}
    if ex.shared_blob is not None:
        expect[int(ex.shared_blob.data_ptr())] = T
    assert int(ex.zero.data_ptr()) not in set(blob.tolist()), "an expert outside the union was read"
    assert set(blob.tolist()) == set(expect), "the experts read are not the union"
    one = T == 1
    rows_gu, rows_dn = (16, 32) if one else (32, 64)
    n_gu, n_dn = I // rows_gu, -(-H // rows_dn)
    items_of = lambda cnt: 1 if one else -(-cnt // 4)
    seen = Counter(zip(blob.tolist(), pas.tolist(), tile.tolist()))
    want = {(bb, p, t) for bb in expect for p, nt in ((0, n_gu), (1, n_dn)) for t in range(nt)}
    assert set(seen) == want
    for (bb, p, t), times in seen.items():
        assert times == items_of(expect[bb]), "a tile was streamed more often than its items"
    assert np.all(rows[pas == 0] == rows_gu) and np.all(rows[pas == 1] == rows_dn)
    # every workgroup walks its rows once (its item has at most 4 tokens)
    assert np.all(walks == 1), np.unique(walks)
    return len(expect)


def test_decode_token_reads_its_nine_experts_once(coli):
    """One GLM-shaped decode token (routing folded into the gate/up pass)."""
    shape = coli.MoEShape(6144, 2048, 256, 1, 8, 0)
    recs, n, idx_ref, ex = _logged_layer(coli, shape, 1, 21, "router")
    assert _check_union_read_once(shape, 1, recs, idx_ref, ex) == 9
    assert n == 9 * (2048 // 16 + 6144 // 32)


def test_mtp_verify_batch_reads_each_unique_expert_once(coli):
    """An 8-token gs64 verify batch with Zipf routing: the union of the 64
    assignments is read once, whatever number of tokens share an expert."""
    shape = coli.MoEShape(6144, 2048, 256, 1, 8, 64)
    recs, n, idx_ref, ex = _logged_layer(coli, shape, 8, 22, "zipf")
    u = _check_union_read_once(shape, 8, recs, idx_ref, ex)
    assert u - 1 == len(np.unique(idx_ref)) < 64          # tokens do share experts
    _, cnt = np.unique(idx_ref, return_counts=True)
    items = int(sum(-(-c // 4) for c in cnt)) + 2         # the shared expert: 8 tokens, 2 items
    assert (cnt > 4).any() and n == items * (2048 // 32 + 6144 // 64)


@pytest.mark.parametrize("T,E,k,n_shared,seed", [(3, 16, 4, 0, 23), (13, 32, 4, 1, 24),
                                                 (2, 8, 8, 1, 25)])
def test_small_batches_read_union_once(coli, T, E, k, n_shared, seed):
    """Batches of a small layer: no shared expert, a token count that splits
    experts into items of 4 tokens and a remainder, and every expert selected
    by both tokens."""
    shape = coli.MoEShape(512, 256, E, n_shared, k, 0)
    recs, _, idx_ref, ex = _logged_layer(coli, shape, T, seed, "zipf")
    _check_union_read_once(shape, T, recs, idx_ref, ex)


def test_adaptive_topp_skips_dropped_experts(coli):
    """With the adaptive top-p, the experts of dropped slots are not read."""
    shape = coli.MoEShape(512, 256, 64, 1, 8, 0, topp=0.5)
    recs, _, idx_ref, ex = _logged_layer(coli, shape, 1, 26, "zipf", topp=0.5)
    assert (idx_ref < 0).any()
    _check_union_read_once(shape, 1, recs, idx_ref, ex)


def test_log_overflow_counts_on(coli):
    """A log smaller than the launch keeps counting and writes only its capacity."""
    shape = coli.MoEShape(512, 256, 16, 1, 4, 0)
    recs, n, _, _ = _logged_layer(coli, shape, 1, 27, "zipf", cap=3)
    assert len(recs) == 3 and n == 5 * (256 // 16 + 512 // 32)
