"""Benchmark: one GLM-5.2-shaped int4 MoE layer on one MI355X.

Default workload (the headline): batch-1 decode, hidden 6144, inter 2048, 256
routed + 1 shared experts, top-8 sigmoid routing from an f32 router, per-row
int4 scales, all 257 expert blobs (4.86 GB) resident in HBM, 1,000 seeded
tokens. A step is one token through the whole layer (router logits, route,
union, gate/up GEMV, down GEMV, combine); steps run back to back on one stream
(replayed from a HIP graph captured over all timed tokens).

Prints one JSON line: tokens/s, the roofline of the dominant kernel (gate/up
GEMV, HIP-event timed on its own stream inside the timed region) and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed tokens (default 1000; 512 for the stream workload)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--graph", type=int, default=1, help="replay the timed tokens from a HIP graph")
    ap.add_argument("--cpu-sample", type=int, default=8, help="tokens of the CPU oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle sample for about this long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--wbits", type=int, default=4, choices=[4, 8],
                    help="decode with int8 experts (8) instead of int4 (4, the headline)")
    ap.add_argument("--topp", type=float, default=0.0,
                    help="decode with the adaptive expert top-p (lossy; 0 = fixed top-8, the headline)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 2048-token prefill line")
    ap.add_argument("--group", type=int, default=0, choices=[0, 64],
                    help="prefill workload: scale group of the experts (0 per-row, 64 gs64)")
    ap.add_argument("--pinned-layers", type=int, default=13,
                    help="stream workload: distinct pinned layer pools (the rest reuse them)")
    ap.add_argument("--policies", default="lru",
                    help="stream workload: comma-separated placement policies, each run on a reset "
                         "cache: lru; pinN (pin the N hottest experts of each layer from a usage "
                         "history of later tokens); repinN (pinN, then repin every --repin-every "
                         "tokens, 4 swaps, 25%% hysteresis, heat decay --repin-decay); lookR "
                         "(lookahead prefetch of the next layer's experts predicted with recall R); "
                         "parts combine with +, e.g. pin48+look1.0")
    ap.add_argument("--repin-every", type=int, default=64)
    ap.add_argument("--repin-decay", type=float, default=0.9)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "mtp", "stream", "copy", "convert"],
                    help="decode (headline, with the prefill line), prefill (that line alone), "
                         "mtp (gs64, 8-token verify batches), stream (16 layers from pinned host through an HBM cache), "
                         "copy (plain 1 GiB device copy: bandwidth and counter calibration), "
                         "convert (FP8 -> int4 conversion of 32 experts)")
    return ap.parse_args()


def build_experts(coli, shape, seed, dev, keep_host=(), layer=0):
    """All routed + shared experts of `layer` quantised on the GPU from seeded
    f32 weights. Returns (arena, table, shared_blob, host f32 copies of
    `keep_host`)."""
    import torch
    import synth
    H, I, E = shape.hidden, shape.inter, shape.n_routed
    nbytes = coli.blob_layout(shape)[1]
    arena = torch.empty((E + 1) * nbytes, dtype=torch.uint8, device=dev)
    g_d = torch.empty((I, H), dtype=torch.float32, device=dev)
    u_d = torch.empty((I, H), dtype=torch.float32, device=dev)
    d_d = torch.empty((H, I), dtype=torch.float32, device=dev)
    g_h = torch.empty((I, H), dtype=torch.float32).pin_memory()
    u_h = torch.empty((I, H), dtype=torch.float32).pin_memory()
    d_h = torch.empty((H, I), dtype=torch.float32).pin_memory()
    kept = {}
    for e in range(E + 1):
        synth.expert_matrix(seed, layer, e, synth.MAT_GATE, I, H, out=g_h.numpy())
        synth.expert_matrix(seed, layer, e, synth.MAT_UP, I, H, out=u_h.numpy())
        synth.expert_matrix(seed, layer, e, synth.MAT_DOWN, H, I, out=d_h.numpy())
        if e in keep_host:
            kept[e] = (g_h.numpy().copy(), u_h.numpy().copy(), d_h.numpy().copy())
        g_d.copy_(g_h, non_blocking=True)
        u_d.copy_(u_h, non_blocking=True)
        d_d.copy_(d_h, non_blocking=True)
        coli.quantize_expert(shape, g_d, u_d, d_d, blob=arena[e * nbytes:(e + 1) * nbytes])
        torch.cuda.synchronize()
        if e % 64 == 0:
            log(f"experts quantised: {e + 1}/{E + 1}")
    blobs = [arena.data_ptr() + e * nbytes for e in range(E)]
    table = coli.blob_table(blobs, dev)
    shared = arena[E * nbytes:(E + 1) * nbytes]
    return arena, table, shared, kept


def cpu_baseline_decode(shape, seed, wr, b, x_all, sample, kept, seconds):
    """The oracle's whole layer on `sample` tokens of the same workload, timed
    over about `seconds` of work."""
    import oracle
    H, I, E, k = shape.hidden, shape.inter, shape.n_routed, shape.top_k
    bits = shape.wbits
    z = np.zeros((I, H), np.float32)
    zero = oracle.QExpert.quantize(z, z, np.zeros((H, I), np.float32), 0, bits=bits)
    experts = [zero] * E
    for e, (g, u, d) in kept.items():
        if e < E:
            experts[e] = oracle.QExpert.quantize(g, u, d, 0, bits=bits)
    shared = oracle.QExpert.quantize(*kept[E], 0, bits=bits)
    x = np.ascontiguousarray(x_all[:sample])
    # the same tokens again until about `seconds` of CPU work (their ~50 experts,
    # about 1 GB of weights, do not stay in the CPU caches between passes)
    reps, dt = 0, 0.0
    t0 = time.perf_counter()
    while dt < seconds and reps < 1000:
        oracle.layer(x, experts, shared, k, 0, 1.0, wr=wr, bias=b, topp=shape.topp)
        reps += 1
        dt = time.perf_counter() - t0
    return {"value": reps * sample / dt, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {sample} tokens of the decode workload, {reps} passes ({reps * sample} "
                      f"token-layers), whole layer (router logits, route, union, 9 expert FFNs, "
                      f"combine), scalar C, f64 accumulation, OpenMP over output rows; {dt:.1f} s"}


def measured_traffic(kernel_json):
    """HBM bytes per launch from the committed counter profile, if the kernel's
    sources are unchanged since the counters were taken (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", kernel_json)
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for f in rec["source_files"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return rec["traffic_bytes_per_dispatch"]
    except (OSError, KeyError, ValueError):
        return None


def sleep_cycles_for(stream, ms):
    """Argument of torch.cuda._sleep (a bounded spin kernel) that holds the
    stream for about `ms` milliseconds, from one timed probe of 2^20 cycles."""
    import torch
    probe = 1 << 20
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(probe)                 # first launch outside the timing
        a.record()
        torch.cuda._sleep(probe)
        b.record()
    b.synchronize()
    per_cycle = max(a.elapsed_time(b), 1e-3) / probe
    return max(1, int(ms / per_cycle))


def run_prefill(coli, shape, table, shared, seed, dev, calls=10, warmup=3):
    """2048-token prefill through the same layer: Zipf(1.1) + 10% uniform
    routing (router logits with that popularity), bf16 MFMA grouped GEMM."""
    import torch
    import synth
    H, I, E, k, T = shape.hidden, shape.inter, shape.n_routed, shape.top_k, 2048
    lg = torch.from_numpy(synth.zipf_logits(seed, 1, 0, T, E, s=1.1, mix=0.1)).to(dev)
    x = torch.from_numpy(synth.activations(seed, 1, 0, T, H)).to(dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    ws = coli.workspace(shape, T, coli.PATH_MFMA, dev)

    def call():
        coli.layer_fwd(shape, x, table=table, shared_blob=shared, logits=lg, y=y, idx_out=idx,
                       path=coli.PATH_MFMA, ws=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    coli.profile_enable(2 * calls + 8)
    t0 = time.perf_counter()
    for _ in range(calls):
        call()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / calls
    n_gu, ms_gu = coli.profile_summary("gemm_gateup")
    n_dn, ms_dn = coli.profile_summary("gemm_down")
    coli.profile_enable(0)
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=E)
    flops_gu = 2.0 * 2 * H * I * (T * k + T)
    flops_dn = 2.0 * H * I * (T * k + T)
    gu_s, dn_s = ms_gu / max(1, n_gu) / 1e3, ms_dn / max(1, n_dn) / 1e3
    used = int((counts > 0).sum()) + shape.n_shared           # experts whose weights the call reads
    weight_bytes = used * coli.blob_layout(shape)[1]
    return {
        "workload": "prefill, 2048 tokens, Zipf(1.1) + 10% uniform routing, same layer"
                    + (", gs64 experts" if shape.group else ""),
        "tokens_per_s": round(T / dt, 1),
        "ms_per_call": round(dt * 1e3, 4),
        "tflops_layer": round((flops_gu + flops_dn) / dt / 1e12, 2),
        "gemm_gateup_us": round(gu_s * 1e6, 2),
        "gemm_down_us": round(dn_s * 1e6, 2),
        "gemm_tflops": round((flops_gu + flops_dn) / (gu_s + dn_s) / 1e12, 2) if n_gu else None,
        "gemm_frac_of_bf16_peak": round((flops_gu + flops_dn) / (gu_s + dn_s) / 1e12 / BF16_PEAK_TFLOPS, 4) if n_gu else None,
        "algorithmic_tflop": round((flops_gu + flops_dn) / 1e12, 4),
        "experts_used": int((counts > 0).sum()),
        # routed experts by tokens routed to them (M), bins [lo, hi)
        "tokens_per_expert_histogram": {f"{lo}-{hi - 1}": int(((counts >= lo) & (counts < hi)).sum())
                                        for lo, hi in ((1, 9), (9, 17), (17, 33), (33, 65), (65, 129),
                                                       (129, 257), (257, 513), (513, T + 1))},
        # every resident weight byte read once per call, over the two GEMMs' time
        "weights_GBps_over_gemm_time": round(weight_bytes / (gu_s + dn_s) / 1e9, 1) if n_gu else None,
        "tokens_per_expert_max": int(counts.max()),
        "tokens_per_expert_median": float(np.median(counts[counts > 0])),
        "tokens_per_expert_min": int(counts[counts > 0].min()),
    }


def run_mtp(args, coli, dev):
    """MTP-verify batches: gs64 scales, 8 tokens per call, router logits with
    Zipf(1.1) popularity (Gumbel top-k), bias 0, 125 calls = 1,000 tokens."""
    import torch
    import synth
    H, I, E, k, T = 6144, 2048, 256, 8, 8
    shape = coli.MoEShape(H, I, E, 1, k, 64, 1.0)
    steps = max(1, args.steps // T)
    warm = max(1, args.warmup // T + 1)
    n = steps + warm
    t0 = time.perf_counter()
    arena, table, shared, _ = build_experts(coli, shape, args.seed, dev)
    log(f"gs64 experts ready in {time.perf_counter() - t0:.1f} s")
    lg = torch.from_numpy(synth.zipf_logits(args.seed, 0, 0, n * T, E, s=1.1)).to(dev)
    x = torch.from_numpy(synth.activations(args.seed, 0, 0, n * T, H)).to(dev)
    y = torch.empty((n * T, H), dtype=torch.float32, device=dev)
    idx = torch.empty((n * T, k), dtype=torch.int32, device=dev)
    ws = coli.workspace(shape, T, coli.PATH_GEMV, dev)
    stream = torch.cuda.Stream()

    def call(i):
        sl = slice(i * T, (i + 1) * T)
        coli.layer_fwd(shape, x[sl], table=table, shared_blob=shared, logits=lg[sl], y=y[sl],
                       idx_out=idx[sl], path=coli.PATH_GEMV, ws=ws)

    with torch.cuda.stream(stream):
        for i in range(warm):
            call(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(warm, n):
            call(i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    coli.profile_enable(2 * steps + 8)
    with torch.cuda.stream(stream):
        for i in range(warm, n):
            call(i)
    torch.cuda.synchronize()
    n_gu, ms_gu = coli.profile_summary("gemv_gateup")
    n_dn, ms_dn = coli.profile_summary("gemv_down")
    coli.profile_enable(0)
    ids = idx[warm * T:].cpu().numpy().reshape(steps, T * k)
    uniq = np.array([len(np.unique(r)) for r in ids])
    blob = coli.blob_layout(shape)[1]
    off, _ = coli.blob_layout(shape)
    gu_bytes = (uniq + 1) * (off[2] - off[0] + (off[5] - off[3]))      # gate/up nibbles + scales
    dn_bytes = (uniq + 1) * (off[3] - off[2] + (blob - off[5]))        # down nibbles + scales
    gu_s = ms_gu / max(1, n_gu) / 1e3
    dn_s = ms_dn / max(1, n_dn) / 1e3
    gbps = float((gu_bytes + dn_bytes).mean()) / (gu_s + dn_s) / 1e9
    tok_s = steps * T / elapsed
    return {
        "metric": "MTP-verify tokens/s (gs64, 8-token batches; weight GB/s vs HBM peak)",
        "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": round(1e3 * elapsed / steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 weights (gs64) x f32 activations (exact int32 nibble products), f32 accumulate",
        "data": "synthetic (seeded Philox N(0,0.02) weights, N(0,1) activations, Zipf(1.1) logits)",
        "config": {"workload": "MTP-verify batches of 8 tokens, GLM-5.2-shaped layer, gs64",
                   "hidden": H, "inter": I, "n_routed": E, "top_k": k, "group": 64,
                   "tokens": steps * T, "graph": True},
        "unique_experts_per_token": round(float(uniq.mean()) / T, 3),
        "unique_experts_per_step_mean": round(float(uniq.mean()), 2),
        "unique_experts_per_step_range": [int(uniq.min()), int(uniq.max())],
        "roofline": {"bound": "hbm", "kernel": "gemv_gateup + gemv_down",
                     "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "avg_gateup_us": round(gu_s * 1e6, 2), "avg_down_us": round(dn_s * 1e6, 2)},
    }


def run_stream(args, coli, dev):
    """Streaming decode across 16 layers: 16 x 256 expert blobs (77.5 GB) in
    pinned host memory, an HBM LRU cache of 64 experts per layer, routing with
    temporal locality (each of the previous token's experts kept with p = 0.6,
    the rest drawn by Zipf(1.1) popularity), batch 1, 512 tokens."""
    import torch
    import synth
    H, I, E, k, L, S = 6144, 2048, 256, 8, 16, 64
    n_tok = max(1, args.steps)
    shape = coli.MoEShape(H, I, E, 1, k, 0, 1.0)
    blob = coli.blob_layout(shape)[1]
    t0 = time.perf_counter()
    arena0, _, shared0, _ = build_experts(coli, shape, args.seed, dev)
    # one pinned pool per layer; pinned host memory per process is capped (near
    # 64 GiB where measured: 13 layer pools of 4.84 GB fit with headroom), so the
    # last layers stream from the pools of the first ones (same copies, same traffic)
    n_pools = min(L, args.pinned_layers)
    log(f"layer-0 experts ready in {time.perf_counter() - t0:.1f} s; pinning {n_pools} x {E * blob / 1e9:.2f} GB")
    t0 = time.perf_counter()
    pools = []
    for l in range(n_pools):
        p = pinned_bytes(E * blob)
        # layer l holds the layer-0 experts in a seeded order of its own
        order = synth.permutation(args.seed, synth.TAG_PERM, 1000 + l, 0, E)
        for e in range(E):
            src = int(order[e])
            p[e * blob:(e + 1) * blob].copy_(arena0[src * blob:(src + 1) * blob])
        pools.append(p)
        log(f"host pool: layer {l + 1}/{n_pools} filled")
    layer_pools = [pools[l % n_pools] for l in range(L)]
    log(f"host pool filled in {time.perf_counter() - t0:.1f} s")
    shared = [shared0.clone() for _ in range(L)]
    del arena0
    arena = torch.empty(L * S * blob, dtype=torch.uint8, device=dev)
    copy_stream = torch.cuda.Stream()
    cache = coli.ExpertCache(L, E, S, blob, arena=arena, pools=layer_pools, copy_stream=copy_stream)
    # routing of the timed tokens, plus as many later tokens of the same process
    # whose picks serve as a usage history from an earlier session
    loc = [synth.locality_logits(args.seed, l, 2 * n_tok, E, k, keep_p=0.6) for l in range(L)]
    lg = [torch.from_numpy(np.ascontiguousarray(loc[l][0][:n_tok])).to(dev) for l in range(L)]
    chosen = [loc[l][1][:n_tok] for l in range(L)]
    history = np.zeros((L, E), np.uint64)
    for l in range(L):
        for row in loc[l][1][n_tok:]:
            history[l, row] += 1
    xs = [torch.from_numpy(synth.activations(args.seed, l, 0, n_tok, H)).to(dev) for l in range(L)]
    y = torch.empty((1, H), dtype=torch.float32, device=dev)
    ws = coli.workspace(shape, 1, coli.PATH_GEMV, dev)
    cold = min(16, n_tok)

    def guesses(recall):
        """Lookahead predictions of every (layer, token): each true pick kept with
        probability `recall`, otherwise replaced by an expert outside the set."""
        rng = np.random.default_rng(args.seed + 7)
        out = []
        for l in range(L):
            g = chosen[l].copy()
            for t in range(n_tok):
                for j in range(k):
                    if rng.random() >= recall:
                        while True:
                            e = int(rng.integers(E))
                            if e not in chosen[l][t] and e not in g[t]:
                                break
                        g[t, j] = e
            out.append(g)
        return out

    def run_policy(policy):
        cache.reset()
        pin_n, repin, recall = 0, False, None
        for part in policy.split("+"):
            if part.startswith("pin"):
                pin_n = int(part[3:])
            elif part.startswith("repin"):
                pin_n, repin = int(part[5:]), True
            elif part.startswith("look"):
                recall = float(part[4:])
            elif part != "lru":
                raise ValueError(f"unknown placement policy {part}")
        guess = guesses(recall) if recall is not None else None
        if pin_n:
            cache.pin_hot(pin_n, history)
        torch.cuda.synchronize()
        st0 = cache.stats()
        coli.profile_enable(2 * L * n_tok + 8)
        t_start = time.perf_counter()
        t_cold, st_cold = None, None
        for t in range(n_tok):
            if repin and t > 0 and t % args.repin_every == 0:
                cache.repin(4, 0.25, args.repin_decay)
            for l in range(L):
                coli.layer_fwd(shape, xs[l][t:t + 1], shared_blob=shared[l],
                               logits=lg[l][t:t + 1], cache=cache, layer=l, y=y,
                               path=coli.PATH_GEMV, ws=ws)
                if guess is not None:
                    # the next layer call's experts, predicted, copied during this one's
                    nl, nt = (l + 1, t) if l + 1 < L else (0, t + 1)
                    if nt < n_tok:
                        cache.prefetch(nl, guess[nl][nt])
            if t + 1 == cold:
                torch.cuda.synchronize()
                t_cold = time.perf_counter()
                st_cold = cache.stats()
        torch.cuda.synchronize()
        t_end = time.perf_counter()
        n_gu, ms_gu = coli.profile_summary("gemv_gateup")
        n_dn, ms_dn = coli.profile_summary("gemv_down")
        coli.profile_enable(0)
        st = cache.stats()
        warm_tok = n_tok - cold
        d = {key: st[key] - st_cold[key] for key in st}
        lookups_w = d["hits"] + d["misses"]
        pcie = (st["bytes_h2d"] - st0["bytes_h2d"]) / max(1, st["copy_ns"] - st0["copy_ns"])
        # 9 blobs per layer call, over the GEMV kernels' summed time (a cached call
        # launches each GEMV twice: resident experts, then the copied ones)
        ffn_bytes = 9 * blob * L * n_tok
        hbm = ffn_bytes / ((ms_gu + ms_dn) / 1e3) / 1e9 if n_gu else None
        warm_s = t_end - t_cold if warm_tok else None
        log(f"stream policy {policy}: {warm_tok / warm_s if warm_tok else 0:.1f} tokens/s warm")
        return {
            "policy": policy,
            "tokens_per_s_warm": round(warm_tok / warm_s, 3) if warm_tok else None,
            "ms_per_token_warm": round(1e3 * warm_s / warm_tok, 4) if warm_tok else None,
            "cold_tokens_per_s": round(cold / (t_cold - t_start), 3),
            "hit_rate_warm": round(d["hits"] / max(1, lookups_w), 4),
            "misses_per_token_per_layer_warm": round(d["misses"] / max(1, warm_tok * L), 3),
            "copies_per_token_per_layer_warm": round(d["bytes_h2d"] / blob / max(1, warm_tok * L), 3),
            "pcie_GBps": round(pcie, 2), "h2d_GB": round((st["bytes_h2d"] - st0["bytes_h2d"]) / 1e9, 2),
            "hbm_GBps_ffn_kernels": round(hbm, 1) if hbm else None,
            "cache": st,
        }

    results = [run_policy(p) for p in args.policies.split(",")]
    cache.close()
    main = results[0]
    return {
        "metric": "streaming decode tokens/s, 16 layers, experts streamed from pinned host (hit rate, PCIe and HBM GB/s)",
        "value": main["tokens_per_s_warm"], "unit": "tokens/s",
        "n_gpus": 1, "steps": n_tok - cold, "warmup": cold,
        "ms_per_step": main["ms_per_token_warm"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 weights x f32 activations (exact int32 nibble products), f32 accumulate",
        "data": "synthetic (seeded Philox weights; layer l holds the layer-0 experts in a seeded order; locality routing)",
        "config": {"workload": "streaming decode, 16 GLM-5.2-shaped layers, 64-slot HBM cache per layer",
                   "hidden": H, "inter": I, "n_routed": E, "top_k": k, "layers": L, "slots": S,
                   "host_pool_GB": round(L * E * blob / 1e9, 2),
                   "distinct_pinned_pools": n_pools, "tokens": n_tok, "policy": main["policy"]},
        **{key: v for key, v in main.items() if key != "policy"},
        "policies": results[1:],
    }


def run_convert(args, coli, dev):
    """FP8 -> int4 conversion of GLM-5.2-shaped experts (hidden 6144, inter
    2048): e4m3 codes with one scale per 128 x 128 block, as in the FP8
    checkpoint, into per-row int4 blobs. 32 expert inputs resident in HBM (4
    distinct generated ones, copied), converted K times."""
    import torch
    import synth
    H, I, n_exp = 6144, 2048, 32
    shape = coli.MoEShape(H, I, 256, 1, 8, 0)
    blob_bytes = coli.blob_layout(shape)[1]
    base = []
    for e in range(4):
        mats = [synth.fp8_block_matrix(args.seed, 0, e, m, r, c)
                for m, (r, c) in ((synth.MAT_GATE, (I, H)), (synth.MAT_UP, (I, H)),
                                  (synth.MAT_DOWN, (H, I)))]
        base.append([torch.from_numpy(a).to(dev) for pair in mats for a in pair])
    inputs = [[t.clone() for t in base[e % 4]] for e in range(n_exp)]
    blobs = torch.empty((n_exp, blob_bytes), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()

    def step():
        for e in range(n_exp):
            coli.convert_fp8_expert(shape, *inputs[e], blob=blobs[e], stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup)):
            step()
    torch.cuda.synchronize()
    k = max(1, min(args.steps, 50))
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        t0.record(stream)
        for _ in range(k):
            step()
        t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / k
    in_bytes = sum(t.numel() * t.element_size() for t in inputs[0])
    per_expert = in_bytes + blob_bytes
    gbps = per_expert * n_exp / (ms / 1e3) / 1e9
    # the f32 quantiser on the same experts' f32 weights (8 resident experts)
    del inputs
    f32 = [[torch.from_numpy(a).to(dev) for a in synth.expert_weights(args.seed, 0, e, H, I)]
           for e in range(8)]
    with torch.cuda.stream(stream):
        for e in range(8):
            coli.quantize_expert(shape, *f32[e], blob=blobs[e], stream=stream)
        t0.record(stream)
        for _ in range(k):
            for e in range(8):
                coli.quantize_expert(shape, *f32[e], blob=blobs[e], stream=stream)
        t1.record(stream)
    torch.cuda.synchronize()
    ms_q = t0.elapsed_time(t1) / k / 8
    q_bytes = sum(t.numel() * 4 for t in f32[0]) + blob_bytes
    return {
        "metric": "FP8 -> int4 expert conversion (GB/s of FP8 read + int4 written)",
        "value": round(n_exp / (ms / 1e3), 1), "unit": "experts/s", "n_gpus": 1, "steps": k,
        "warmup": max(1, args.warmup), "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "e4m3 -> f32 -> int4 (per-row scales)",
        "data": "synthetic checkpoint-style FP8 (N(0, 0.02) weights, block max / 448 scales)",
        "config": {"workload": f"FP8 -> int4 conversion of {n_exp} GLM-5.2-shaped experts per step",
                   "hidden": H, "inter": I, "experts_per_step": n_exp},
        "roofline": {"bound": "hbm", "kernel": "fp8_wave_kernel (3 launches per expert)",
                     "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_expert": per_expert},
        "quantize_f32": {"experts_per_s": round(1e3 / ms_q, 1), "us_per_expert": round(ms_q * 1e3, 2),
                         "GBps": round(q_bytes / (ms_q / 1e3) / 1e9, 1), "bytes_per_expert": q_bytes},
    }


def run_copy(args, dev):
    """A plain device-to-device copy of 1 GiB, 20 times: the achievable
    read+write bandwidth, and the reference for scaling HBM byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(20):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    s = a.elapsed_time(b) / 1e3 / 20
    return {"metric": "device copy GB/s (read + write)", "value": round(2 * n / s / 1e9, 1),
            "unit": "GB/s", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
            "us_per_copy": round(s * 1e6, 2), "n_gpus": 1}


def pinned_bytes(nbytes):
    """Exactly `nbytes` of pinned host memory (hipHostMalloc) as a uint8 tensor;
    torch's pinned allocator would round a 77.5 GB request up to a power of two."""
    import ctypes
    import torch
    hip = ctypes.CDLL("libamdhip64.so")
    ptr = ctypes.c_void_p()
    rc = hip.hipHostMalloc(ctypes.byref(ptr), ctypes.c_size_t(nbytes), ctypes.c_uint(0))
    if rc != 0 or not ptr.value:
        raise RuntimeError(f"hipHostMalloc of {nbytes} bytes failed ({rc})")
    buf = (ctypes.c_uint8 * nbytes).from_address(ptr.value)
    t = torch.frombuffer(buf, dtype=torch.uint8)
    t._coli_keep = (hip, ptr, buf)
    return t


def main():
    args = parse()
    if args.steps is None:
        args.steps = 512 if args.workload == "stream" else 1000
    if args.gpus != 1:
        print(json.dumps({"error": "one-GPU benchmark: the layer runs on a single GPU here (how it would shard is described, not run); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import synth
    import int4_routed_expert_sigmoid_amd as coli
    import oracle

    dev = torch.device("cuda:0")
    if args.workload != "decode":
        if args.workload == "copy":
            line = run_copy(args, dev)
        elif args.workload == "prefill":
            shape = coli.MoEShape(6144, 2048, 256, 1, 8, args.group, 1.0)
            arena, table, shared, _ = build_experts(coli, shape, args.seed, dev)
            line = run_prefill(coli, shape, table, shared, args.seed, dev,
                               calls=max(1, min(args.steps, 50)), warmup=max(1, args.warmup))
            line = {"metric": "prefill TFLOP/s (2048 tokens, bf16 MFMA)", "value": line["tflops_layer"],
                    "unit": "TFLOP/s", "n_gpus": 1, **line}
        elif args.workload == "mtp":
            line = run_mtp(args, coli, dev)
        elif args.workload == "convert":
            line = run_convert(args, coli, dev)
        else:
            line = run_stream(args, coli, dev)
        print(json.dumps(line), flush=True)
        return
    H, I, E, k = 6144, 2048, 256, 8
    shape = coli.MoEShape(H, I, E, 1, k, 0, 1.0, args.topp, args.wbits)
    seed = args.seed
    n_tok = args.warmup + args.steps
    log(f"decode workload: {n_tok} tokens, H={H} I={I} E={E}+1 k={k} topp={args.topp}")

    wr = synth.router_weights(seed, 0, E, H)
    b = synth.bias(seed, 0, E)
    x_all = synth.activations(seed, 0, 0, n_tok, H)
    sample = 0 if args.no_cpu_baseline else min(args.cpu_sample, n_tok)
    keep = set()
    if sample:
        idx_s, _ = oracle.route(oracle.router_logits(wr, x_all[:sample]), b, k)
        keep = set(np.unique(idx_s).tolist()) | {E}
    t0 = time.perf_counter()
    arena, table, shared, kept = build_experts(coli, shape, seed, dev, keep)
    log(f"experts ready in {time.perf_counter() - t0:.1f} s")

    wr_d = torch.from_numpy(wr).to(dev)
    b_d = torch.from_numpy(b).to(dev)
    x_d = torch.from_numpy(x_all).to(dev)
    y_d = torch.empty((n_tok, H), dtype=torch.float32, device=dev)
    idx_d = torch.empty((n_tok, k), dtype=torch.int32, device=dev)
    ws = coli.workspace(shape, 1, coli.PATH_GEMV, dev)

    stream = torch.cuda.Stream()
    # one call per token with the fixed arguments prepared once (the eager
    # pass below then keeps the GPU busy instead of waiting on the host)
    call = coli.LayerCall(shape, 1, ws, table=table, shared_blob=shared, router_w=wr_d, bias=b_d,
                          path=coli.PATH_GEMV, stream=stream)
    xp, yp, ip = x_d.data_ptr(), y_d.data_ptr(), idx_d.data_ptr()

    def token(t):
        call(xp + t * H * 4, yp + t * H * 4, ip + t * k * 4)

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            token(t)
    torch.cuda.synchronize()

    # timed region 1: the K tokens replayed from one HIP graph (how a decode
    # loop is deployed); gives `value`
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for t in range(args.warmup, n_tok):
                token(t)
        torch.cuda.synchronize()
        graph.replay()                      # first replay uploads the graph
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        elapsed_graph = time.perf_counter() - t0
    # timed region 2: the same K tokens launched eagerly, with HIP events
    # attached to each GEMV kernel's dispatch on the stream it runs on (HIP
    # cannot time events recorded inside a captured graph). The host issues a
    # token more slowly than the GPU runs it, so each chunk of tokens is queued
    # behind a short GPU sleep (a bounded spin kernel, longer than the host
    # needs to queue the chunk): the timed kernels then run back to back, as
    # in the graph, instead of each starting on an idle GPU.
    chunk = 100
    sleep_cycles = sleep_cycles_for(stream, chunk * 0.08)      # 80 us of host time per token
    coli.profile_enable(2 * args.steps + 16)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for c0 in range(args.warmup, n_tok, chunk):
            torch.cuda._sleep(sleep_cycles)
            for t in range(c0, min(c0 + chunk, n_tok)):
                token(t)
    torch.cuda.synchronize()
    n_gu, ms_gu = coli.profile_summary("gemv_gateup")
    n_dn, ms_dn = coli.profile_summary("gemv_down")
    coli.profile_enable(0)
    if graph is None:                       # --graph 0: plain eager timing for `value`
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for t in range(args.warmup, n_tok):
                token(t)
        torch.cuda.synchronize()
        elapsed_graph = time.perf_counter() - t0
    elapsed = elapsed_graph

    # algorithmic bytes per token: the routed experts the token uses (8, fewer
    # with top-p: their mean over the timed tokens) and the shared one
    routed = (idx_d[args.warmup:] >= 0).sum(dim=1).double().mean().item()
    n_exp = routed + 1.0
    wb = args.wbits // 4                      # bytes per two weights
    gu_bytes = n_exp * (2 * I * (H * wb // 2) + 2 * I * 4)
    dn_bytes = n_exp * (H * (I * wb // 2) + H * 4)
    gu_avg_s = ms_gu / max(1, n_gu) / 1e3
    dn_avg_s = ms_dn / max(1, n_dn) / 1e3
    gu_gbps = gu_bytes / gu_avg_s / 1e9 if n_gu else None
    dn_gbps = dn_bytes / dn_avg_s / 1e9 if n_dn else None
    gemv_gbps = (gu_bytes + dn_bytes) / (gu_avg_s + dn_avg_s) / 1e9 if n_gu and n_dn else None
    tok_s = args.steps / elapsed

    prefill = None
    if not args.no_prefill and args.wbits == 4:           # the MFMA path is int4 only
        log("prefill: 2048 tokens through the same layer (bf16 MFMA)")
        prefill = run_prefill(coli, shape, table, shared, seed, dev)

    cpu = None
    if sample:
        cpu = cpu_baseline_decode(shape, seed, wr, b, x_all, sample, kept, args.cpu_seconds)

    line = {
        "metric": "MoE-layer tokens/s at decode (int4 weight GB/s vs HBM peak) + prefill TFLOP/s",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"int{args.wbits} weights x f32 activations (exact int32 nibble products), f32 accumulate",
        "data": "synthetic (seeded Philox N(0,0.02) weights, N(0,1) activations, f32 router)",
        "config": {"workload": "GLM-5.2-shaped MoE layer, batch-1 decode"
                               + (f", adaptive expert top-p {args.topp}" if args.topp else "")
                               + (", int8 experts" if args.wbits == 8 else ""),
                   "hidden": H,
                   "inter": I, "n_routed": E, "n_shared": 1, "top_k": k, "group": 0,
                   "wbits": args.wbits,
                   "tokens": args.steps, "graph": bool(args.graph), "topp": args.topp,
                   "routed_experts_per_token": round(routed, 4)},
        "roofline": {"bound": "hbm", "kernel": "gemv_gateup",
                     "achieved": round(gu_gbps, 1) if gu_gbps else None,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gu_gbps / HBM_PEAK_GBPS, 4) if gu_gbps else None,
                     "traffic": (measured_traffic("gemv_gateup_decode_traffic.json")
                                 if args.topp == 0.0 and args.wbits == 4 else None),
                     "bytes_per_launch": round(gu_bytes), "avg_launch_us": round(gu_avg_s * 1e6, 3),
                     "launches_timed": n_gu},
        "expert_gemv": {"gateup_GBps": gu_gbps and round(gu_gbps, 1),
                        "down_GBps": dn_gbps and round(dn_gbps, 1),
                        "both_GBps": gemv_gbps and round(gemv_gbps, 1),
                        "down_avg_us": round(dn_avg_s * 1e6, 3)},
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
