"""Benchmark: one GLM-5.2-shaped int4 MoE layer on one MI355X.

Default workload (the headline): batch-1 decode, hidden 6144, inter 2048, 256
routed + 1 shared experts, top-8 sigmoid routing from an f32 router, per-row
int4 scales, all 257 expert blobs (4.86 GB) resident in HBM, 1,000 seeded
tokens. Every token is one pass of the whole layer (router logits, route,
union, gate/up GEMV, down GEMV, combine), run back to back on one stream. A
step is one pass over the 1,000-token workload, replayed from a HIP graph
captured over all of its tokens; --steps K times K replays.

Prints one JSON line: tokens/s, the roofline of the dominant kernel (gate/up
GEMV: graph-replayed back-to-back launches timed with HIP events on their
stream, with the shared expert and router read from memory that the MALL no
longer holds, and the same warm), a parity check of the timed outputs against
the CPU oracle, and the oracle itself timed on a bounded sample.
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
N_ROTATE = 14          # copies of the shared expert and router for the cold-MALL runs


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps: decode, replays of the 1,000-token workload (default 10); "
                         "mtp, 8-token verify batches (125); stream, tokens (512); prefill and "
                         "convert, calls (10)")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--tokens", type=int, default=1000, help="decode: tokens of the workload")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--mall", default="cold", choices=["cold", "warm"],
                    help="decode headline: cold, the shared expert and router rotate over "
                         f"{N_ROTATE} copies so the MALL holds none of them when a token reads "
                         "them (as in a model of many layers); warm, one copy, re-read every token")
    ap.add_argument("--parity-tokens", type=int, default=64,
                    help="timed outputs compared with the oracle (routing: every token)")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=8, help="tokens of the CPU oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle sample for about this long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--wbits", type=int, default=4, choices=[4, 8],
                    help="decode with int8 experts (8) instead of int4 (4, the headline)")
    ap.add_argument("--topp", type=float, default=0.0,
                    help="decode with the adaptive expert top-p (lossy; 0 = fixed top-8, the headline)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 2048-token prefill line")
    ap.add_argument("--prefill-mix", type=float, default=0.1,
                    help="prefill routing: share of uniform popularity mixed with Zipf(1.1) (0.1 is "
                         "the workload; 1.0 spreads the 2048 tokens evenly, about 64 per expert)")
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
                    choices=["decode", "prefill", "mtp", "stream", "copy", "convert", "readprobe"],
                    help="decode (headline, with the prefill line), prefill (that line alone), "
                         "mtp (gs64, 8-token verify batches), stream (16 layers from pinned host through an HBM cache), "
                         "copy (plain 1 GiB device copy: bandwidth and counter calibration), "
                         "readprobe (read-only streaming kernels in the decode GEMVs' access patterns: "
                         "the practical HBM read ceiling of each), "
                         "convert (FP8 -> int4 conversion of 32 experts)")
    return ap.parse_args()


def spread(n, count):
    """`count` indices spread evenly over range(n)."""
    return np.unique(np.linspace(0, n - 1, min(n, count)).round().astype(int))


def rel_l2_rows(y, ref):
    a = np.asarray(y, np.float64)
    b = np.asarray(ref, np.float64)
    den = np.linalg.norm(b, axis=1)
    return np.linalg.norm(a - b, axis=1) / np.where(den > 0, den, 1.0)


def build_experts(coli, shape, seed, dev, oracle_ids=(), layer=0):
    """All routed + shared experts of `layer` quantised on the GPU from seeded
    f32 weights. The experts in `oracle_ids` are also quantised by the oracle
    from the same f32 weights. Returns (arena, table, shared_blob, {id: oracle
    expert})."""
    import torch
    import oracle
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
    qx = {}
    for e in range(E + 1):
        synth.expert_matrix(seed, layer, e, synth.MAT_GATE, I, H, out=g_h.numpy())
        synth.expert_matrix(seed, layer, e, synth.MAT_UP, I, H, out=u_h.numpy())
        synth.expert_matrix(seed, layer, e, synth.MAT_DOWN, H, I, out=d_h.numpy())
        g_d.copy_(g_h, non_blocking=True)
        u_d.copy_(u_h, non_blocking=True)
        d_d.copy_(d_h, non_blocking=True)
        coli.quantize_expert(shape, g_d, u_d, d_d, blob=arena[e * nbytes:(e + 1) * nbytes])
        if e in oracle_ids:             # the CPU quantises while the GPU works
            qx[e] = oracle.QExpert.quantize(g_h.numpy(), u_h.numpy(), d_h.numpy(), shape.group,
                                            bits=shape.wbits)
        torch.cuda.synchronize()
        if e % 64 == 0:
            log(f"experts quantised: {e + 1}/{E + 1}")
    blobs = [arena.data_ptr() + e * nbytes for e in range(E)]
    table = coli.blob_table(blobs, dev)
    shared = arena[E * nbytes:(E + 1) * nbytes]
    return arena, table, shared, qx


def oracle_list(qx, shape):
    """Oracle experts [E] (ids without a copy get one all-zero expert) and the shared one."""
    import oracle
    H, I, E = shape.hidden, shape.inter, shape.n_routed
    z = np.zeros((I, H), np.float32)
    zero = oracle.QExpert.quantize(z, z, np.zeros((H, I), np.float32), shape.group,
                                   bits=shape.wbits)
    return [qx.get(e, zero) for e in range(E)], qx[E]


def check_outputs(y_gpu, y_ref64, tol):
    err = rel_l2_rows(y_gpu, y_ref64)
    return {"y_tokens_checked": int(len(err)), "y_max_rel_l2": float(f"{err.max():.3e}"),
            "y_tol": tol, "y_pass": bool(err.max() <= tol)}


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


def time_replays(graph, stream, n):
    """Milliseconds of each of n replays, HIP events on the graph's stream."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    with torch.cuda.stream(stream):
        evs[0].record(stream)
        for i in range(n):
            graph.replay()
            evs[i + 1].record(stream)
    evs[-1].synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]


def cpu_baseline(coli_shape, x, oracle_args, seconds, label):
    """The oracle's whole layer on the sample x, repeated for about `seconds`
    on every core, then one pass over two tokens on one core (extrapolated)."""
    import oracle
    threads = oracle.num_threads()
    reps, dt = 0, 0.0
    t0 = time.perf_counter()
    while dt < seconds and reps < 1000:
        oracle.layer(x, **oracle_args)
        reps += 1
        dt = time.perf_counter() - t0
    oracle.set_num_threads(1)
    try:
        n1 = min(2, len(x))
        t1 = time.perf_counter()
        oracle.layer(np.ascontiguousarray(x[:n1]), **oracle_args)
        dt1 = time.perf_counter() - t1
    finally:
        oracle.set_num_threads(threads)
    return {"value": reps * len(x) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(x)} tokens of the {label} workload spread over the run, {reps} passes "
                      f"({reps * len(x)} token-layers), whole layer (router logits, route, union, "
                      f"9 expert FFNs, combine), scalar C, f64 accumulation, OpenMP over output "
                      f"rows; {dt:.1f} s",
            "one_core": {"value": round(n1 / dt1, 4), "unit": "tokens/s", "cores": 1,
                         "kind": "oracle, extrapolated",
                         "sample": f"{n1} tokens once on one thread ({dt1:.2f} s)"}}


def gemv_graph_rates(coli, shape, table, shared_of, wr_of, bias, x_d, tokens, stream, replays):
    """Back-to-back graph-replayed launches of each GEMV pass. Every token is
    first run once through the layer with a workspace of its own (shared expert
    and router copy shared_of(t), wr_of(t)); then a graph of `tokens`
    gate/up launches (coli_profile_rerun), one per token's workspace, and one
    of the down launches are each replayed `replays` times, timed with HIP
    events on their stream. Returns (gate/up us, down us) per launch (median
    replay / tokens)."""
    import torch
    H = shape.hidden
    nb = coli.workspace_size(shape, 1, coli.PATH_GEMV)
    ws = torch.empty((tokens, nb), dtype=torch.uint8, device=x_d.device)
    y = torch.empty((1, H), dtype=torch.float32, device=x_d.device)
    with torch.cuda.stream(stream):
        for t in range(tokens):
            coli.layer_fwd(shape, x_d[t:t + 1], table=table, shared_blob=shared_of(t),
                           router_w=wr_of(t), bias=bias, y=y, path=coli.PATH_GEMV, ws=ws[t],
                           stream=stream)
    torch.cuda.synchronize()
    out = []
    for which in (0, 1):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for t in range(tokens):
                coli.profile_rerun(shape, 1, table, shared_of(t), which, ws[t], stream=stream)
        torch.cuda.synchronize()
        g.replay()                                     # uploads the graph
        torch.cuda.synchronize()
        ms = time_replays(g, stream, replays)
        out.append(float(np.median(ms)) * 1e3 / tokens)
        del g
    del ws
    return out[0], out[1]


def run_decode(args, coli, dev):
    import torch
    import oracle
    import synth
    H, I, E, k = 6144, 2048, 256, 8
    shape = coli.MoEShape(H, I, E, 1, k, 0, 1.0, args.topp, args.wbits)
    seed, N = args.seed, args.tokens
    K, W = args.steps, args.warmup
    log(f"decode workload: {N} tokens per step, {W} + {K} steps, H={H} I={I} E={E}+1 k={k} "
        f"topp={args.topp} wbits={args.wbits}")
    wr = synth.router_weights(seed, 0, E, H)
    b = synth.bias(seed, 0, E)
    x_all = synth.activations(seed, 0, 0, N, H)

    # oracle routing of every token (checked against the timed outputs), and
    # the experts of the sampled tokens, which the oracle also needs
    parity = not args.no_parity
    sample = spread(N, args.parity_tokens)
    need = set()
    if parity or not args.no_cpu_baseline:
        t0 = time.perf_counter()
        idx_ref, w_ref = oracle.route(oracle.router_logits(wr, x_all), b, k, topp=args.topp)
        need |= set(np.unique(idx_ref[sample]).tolist()) - {-1}
        log(f"oracle routing of {N} tokens: {time.perf_counter() - t0:.1f} s")
    with_prefill = not args.no_prefill and args.wbits == 4        # the MFMA path is int4 only
    if with_prefill and parity:
        lgp = synth.zipf_logits(seed, 1, 0, 2048, E, s=1.1, mix=args.prefill_mix)
        need |= set(np.unique(oracle.route(lgp[spread(2048, args.parity_tokens)], None, k)[0]).tolist())
    t0 = time.perf_counter()
    arena, table, shared, qx = build_experts(coli, shape, seed, dev, oracle_ids=need | {E})
    log(f"experts ready in {time.perf_counter() - t0:.1f} s ({len(qx)} also on the oracle side)")

    wr_d = torch.from_numpy(wr).to(dev)
    b_d = torch.from_numpy(b).to(dev)
    x_d = torch.from_numpy(x_all).to(dev)
    # cold-MALL copies of the shared expert and the router: token t reads copy
    # t % N_ROTATE, so between two reads of one copy about 13 tokens' weights
    # (2.3 GB) stream through the 256 MB MALL
    shared_c = [shared] + [shared.clone() for _ in range(N_ROTATE - 1)]
    wr_c = [wr_d] + [wr_d.clone() for _ in range(N_ROTATE - 1)]
    ws = coli.workspace(shape, 1, coli.PATH_GEMV, dev)
    stream = torch.cuda.Stream()
    # one prepared call per copy (the loops below then cost the host little)
    calls = [coli.LayerCall(shape, 1, ws, table=table, shared_blob=shared_c[i], router_w=wr_c[i],
                            bias=b_d, path=coli.PATH_GEMV, stream=stream) for i in range(N_ROTATE)]
    outs = {m: (torch.empty((N, H), dtype=torch.float32, device=dev),
                torch.empty((N, k), dtype=torch.int32, device=dev),
                torch.empty((N, k), dtype=torch.float32, device=dev)) for m in ("cold", "warm")}

    def token(t, mall):
        y_d, idx_d, w_d = outs[mall]
        c = calls[t % N_ROTATE] if mall == "cold" else calls[0]
        c(x_d.data_ptr() + t * H * 4, y_d.data_ptr() + t * H * 4, idx_d.data_ptr() + t * k * 4,
          w_d.data_ptr() + t * k * 4)

    graphs = {}
    for mall in ("cold", "warm"):
        with torch.cuda.stream(stream):
            for t in range(min(N, 16)):
                token(t, mall)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for t in range(N):
                token(t, mall)
        torch.cuda.synchronize()
        graphs[mall] = g
    head, other = args.mall, "warm" if args.mall == "cold" else "cold"

    # timed region: W untimed, then K timed replays of the N-token graph
    for _ in range(max(1, W)):
        graphs[head].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    per_step = time_replays(graphs[head], stream, K)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tok_s = K * N / elapsed
    graphs[other].replay()
    torch.cuda.synchronize()
    per_step_other = time_replays(graphs[other], stream, max(2, K // 4))
    log(f"decode ({head}): {tok_s:.0f} tokens/s; {other}: "
        f"{N / (np.median(per_step_other) / 1e3):.0f} tokens/s")

    # the GEMV kernels: graph-replayed back-to-back launches, cold and warm
    reps = max(3, min(K, 10))
    rot = lambda t: shared_c[t % N_ROTATE]
    rot_wr = lambda t: wr_c[t % N_ROTATE]
    gu_cold, dn_cold = gemv_graph_rates(coli, shape, table, rot, rot_wr, b_d, x_d, N, stream, reps)
    gu_warm, dn_warm = gemv_graph_rates(coli, shape, table, lambda t: shared, lambda t: wr_d, b_d,
                                        x_d, N, stream, reps)
    # and eagerly, with HIP events attached to each dispatch (hipExtLaunchKernel);
    # each chunk of tokens queued behind a short GPU sleep so the launches run
    # back to back as in the graph instead of each starting on an idle GPU
    chunk = 100
    sleep_cycles = sleep_cycles_for(stream, chunk * 0.08)      # 80 us of host time per token
    coli.profile_enable(2 * N + 16)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for c0 in range(0, N, chunk):
            torch.cuda._sleep(sleep_cycles)
            for t in range(c0, min(c0 + chunk, N)):
                token(t, head)
    torch.cuda.synchronize()
    n_gu, ms_gu = coli.profile_summary("gemv_gateup")
    n_dn, ms_dn = coli.profile_summary("gemv_down")
    coli.profile_enable(0)

    y_d, idx_d, w_d = outs[head]
    # algorithmic bytes per token: the routed experts the token uses (8, fewer
    # with top-p: their mean over the tokens) and the shared one
    routed = (idx_d >= 0).sum(dim=1).double().mean().item()
    n_exp = routed + 1.0
    wb = args.wbits // 4                      # bytes per two weights
    gu_bytes = n_exp * (2 * I * (H * wb // 2) + 2 * I * 4)
    dn_bytes = n_exp * (H * (I * wb // 2) + H * 4)
    gbps = lambda nbytes, us: nbytes / (us * 1e-6) / 1e9
    gu_us = gu_cold if head == "cold" else gu_warm
    dn_us = dn_cold if head == "cold" else dn_warm
    eager_gu_us = ms_gu / max(1, n_gu) * 1e3
    eager_dn_us = ms_dn / max(1, n_dn) * 1e3

    result_parity = None
    if parity:
        y_o, idx_o, _ = outs[other]
        torch.cuda.synchronize()
        idx_g = idx_d.cpu().numpy()
        t0 = time.perf_counter()
        experts, sh = oracle_list(qx, shape)
        _, y64, _, _ = oracle.layer(x_all[sample], experts, sh, k, 0, 1.0, wr=wr, bias=b,
                                    topp=args.topp)
        result_parity = {
            "idx_tokens_checked": N,
            "idx_mismatch_tokens": int((idx_g != idx_ref).any(axis=1).sum()),
            "w_mismatch_tokens": int((w_d.cpu().numpy() != w_ref).any(axis=1).sum()),
            **check_outputs(y_d.cpu().numpy()[sample], y64, 1e-3),
            "cold_equals_warm": bool(torch.equal(y_d, y_o) and torch.equal(idx_d, idx_o)),
        }
        result_parity["pass"] = bool(result_parity["idx_mismatch_tokens"] == 0 and
                                     result_parity["w_mismatch_tokens"] == 0 and
                                     result_parity["y_pass"] and result_parity["cold_equals_warm"])
        log(f"parity: {result_parity} ({time.perf_counter() - t0:.1f} s)")

    prefill = None
    if with_prefill:
        log("prefill: 2048 tokens through the same layer (bf16 MFMA)")
        prefill = run_prefill(coli, shape, table, shared, seed, dev,
                              qx=qx if parity else None, parity_tokens=args.parity_tokens,
                              mix=args.prefill_mix)

    cpu = None
    if not args.no_cpu_baseline:
        experts, sh = oracle_list(qx, shape)
        xs = np.ascontiguousarray(x_all[sample[:args.cpu_sample]])
        cpu = cpu_baseline(shape, xs, dict(experts=experts, shared=sh, k=k, group=0,
                                           routed_scale=1.0, wr=wr, bias=b, topp=args.topp),
                           args.cpu_seconds, "decode")

    med = float(np.median(per_step))
    med_other = float(np.median(per_step_other))
    return {
        "metric": "MoE-layer tokens/s at decode (int4 weight GB/s vs HBM peak) + prefill TFLOP/s",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(1e3 * elapsed / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"int{args.wbits} weights x 16-bit block-scaled activations (x and h as four "
                 f"signed base-16 digit planes per 32-element block, one f32 scale per block), "
                 f"exact int32 block sums, f32 accumulate",
        "data": "synthetic (seeded Philox N(0,0.02) weights, N(0,1) activations, f32 router)",
        "config": {"workload": "GLM-5.2-shaped MoE layer, batch-1 decode"
                               + (f", adaptive expert top-p {args.topp}" if args.topp else "")
                               + (", int8 experts" if args.wbits == 8 else ""),
                   "hidden": H, "inter": I, "n_routed": E, "n_shared": 1, "top_k": k, "group": 0,
                   "wbits": args.wbits, "tokens": N, "tokens_per_step": N, "graph": True,
                   "mall": head, "topp": args.topp, "routed_experts_per_token": round(routed, 4)},
        "step_ms": {"median": round(med, 4), "min": round(min(per_step), 4),
                    "max": round(max(per_step), 4), "us_per_token_median": round(med * 1e3 / N, 3)},
        f"{other}_mall": {"tokens_per_s_median": round(N / (med_other / 1e3), 2),
                          "us_per_token_median": round(med_other * 1e3 / N, 3)},
        "roofline": {"bound": "hbm", "kernel": "gemv_gateup",
                     "achieved": round(gbps(gu_bytes, gu_us), 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps(gu_bytes, gu_us) / HBM_PEAK_GBPS, 4),
                     "traffic": (measured_traffic("gemv_gateup_decode_traffic.json")
                                 if args.topp == 0.0 and args.wbits == 4 else None),
                     "traffic_source": "profiles/gemv_gateup_decode_traffic.json (rocprofv3 "
                                       "FETCH_SIZE + WRITE_SIZE, calibrated; null once the "
                                       "kernel's sources change)",
                     "bytes_per_launch": round(gu_bytes), "avg_launch_us": round(gu_us, 3),
                     "timing": f"graph of {N} back-to-back launches (one per token), median of "
                               f"{reps} replays, HIP events on the launch stream, {head} MALL",
                     "graph_frac": round(gbps(gu_bytes, gu_us) / HBM_PEAK_GBPS, 4),
                     "cold_frac": round(gbps(gu_bytes, gu_cold) / HBM_PEAK_GBPS, 4),
                     "warm_frac": round(gbps(gu_bytes, gu_warm) / HBM_PEAK_GBPS, 4),
                     "eager_frac": round(gbps(gu_bytes, eager_gu_us) / HBM_PEAK_GBPS, 4),
                     "eager_avg_launch_us": round(eager_gu_us, 3),
                     "launches_timed": N * reps,
                     # the other expert GEMV and the pair (same timing method)
                     "down_frac": round(gbps(dn_bytes, dn_us) / HBM_PEAK_GBPS, 4),
                     "both_frac": round(gbps(gu_bytes + dn_bytes, gu_us + dn_us) / HBM_PEAK_GBPS, 4)},
        "expert_gemv": {
            "gateup_us": {"cold": round(gu_cold, 3), "warm": round(gu_warm, 3),
                          "eager": round(eager_gu_us, 3)},
            "down_us": {"cold": round(dn_cold, 3), "warm": round(dn_warm, 3),
                        "eager": round(eager_dn_us, 3)},
            "gateup_GBps": round(gbps(gu_bytes, gu_us), 1),
            "down_GBps": round(gbps(dn_bytes, dn_us), 1),
            "down_frac": round(gbps(dn_bytes, dn_us) / HBM_PEAK_GBPS, 4),
            "both_GBps": round(gbps(gu_bytes + dn_bytes, gu_us + dn_us), 1),
            "both_frac": round(gbps(gu_bytes + dn_bytes, gu_us + dn_us) / HBM_PEAK_GBPS, 4),
            "bytes_per_token": round(gu_bytes + dn_bytes)},
        "parity": result_parity,
        "prefill": prefill,
        "cpu_baseline": cpu,
    }


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


def run_prefill(coli, shape, table, shared, seed, dev, calls=10, warmup=3, qx=None,
                parity_tokens=64, mix=0.1):
    """2048-token prefill through the same layer: Zipf(1.1) + 10% uniform
    routing (router logits with that popularity), bf16 MFMA grouped GEMM.
    With oracle experts (qx), the outputs of `parity_tokens` tokens and the
    routing of all are checked against the oracle."""
    import torch
    import oracle
    import synth
    H, I, E, k, T = shape.hidden, shape.inter, shape.n_routed, shape.top_k, 2048
    lg_np = synth.zipf_logits(seed, 1, 0, T, E, s=1.1, mix=mix)
    x_np = synth.activations(seed, 1, 0, T, H)
    lg = torch.from_numpy(lg_np).to(dev)
    x = torch.from_numpy(x_np).to(dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    ws = coli.workspace(shape, T, coli.PATH_AUTO, dev)

    def call():
        # automatic path: bf16 MFMA tiles, experts with at most 4 tokens on the GEMV family
        coli.layer_fwd(shape, x, table=table, shared_blob=shared, logits=lg, y=y, idx_out=idx,
                       path=coli.PATH_AUTO, ws=ws)

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
    n_gv, ms_gv = coli.profile_summary("gemv_gateup")
    n_gd, ms_gd = coli.profile_summary("gemv_down")
    coli.profile_enable(0)
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=E)
    flops_gu = 2.0 * 2 * H * I * (T * k + T)
    flops_dn = 2.0 * H * I * (T * k + T)
    gu_s, dn_s = ms_gu / max(1, n_gu) / 1e3, ms_dn / max(1, n_dn) / 1e3
    gv_s = (ms_gv + ms_gd) / max(1, calls) / 1e3
    used = int((counts > 0).sum()) + shape.n_shared           # experts whose weights the call reads
    weight_bytes = used * coli.blob_layout(shape)[1]
    par = None
    if qx is not None:
        sp = spread(T, parity_tokens)
        idx_ref, _ = oracle.route(lg_np, None, k)
        experts, sh = oracle_list(qx, shape)
        _, y64, _, _ = oracle.layer(x_np[sp], experts, sh, k, shape.group, 1.0, logits=lg_np[sp])
        par = {"idx_tokens_checked": T,
               "idx_mismatch_tokens": int((idx.cpu().numpy() != idx_ref).any(axis=1).sum()),
               **check_outputs(y.cpu().numpy()[sp], y64, 2e-2)}
        par["pass"] = bool(par["idx_mismatch_tokens"] == 0 and par["y_pass"])
        log(f"prefill parity: {par}")
    gemm_s = gu_s + dn_s
    return {
        "workload": f"prefill, 2048 tokens, Zipf(1.1) + {100 * mix:g}% uniform routing, same layer"
                    + (", gs64 experts" if shape.group else ""),
        "tokens_per_s": round(T / dt, 1),
        "ms_per_call": round(dt * 1e3, 4),
        "tflops_layer": round((flops_gu + flops_dn) / dt / 1e12, 2),
        "gemm_gateup_us": round(gu_s * 1e6, 2),
        "gemm_down_us": round(dn_s * 1e6, 2),
        "gemv_small_experts_us": round(gv_s * 1e6, 2) if n_gv else 0.0,
        "gemm_tflops": round((flops_gu + flops_dn) / gemm_s / 1e12, 2) if n_gu else None,
        "gemm_frac_of_bf16_peak": round((flops_gu + flops_dn) / gemm_s / 1e12 / BF16_PEAK_TFLOPS, 4) if n_gu else None,
        "algorithmic_tflop": round((flops_gu + flops_dn) / 1e12, 4),
        "experts_used": int((counts > 0).sum()),
        # routed experts by tokens routed to them (M), bins [lo, hi)
        "tokens_per_expert_histogram": {f"{lo}-{hi - 1}": int(((counts >= lo) & (counts < hi)).sum())
                                        for lo, hi in ((1, 9), (9, 17), (17, 33), (33, 65), (65, 129),
                                                       (129, 257), (257, 513), (513, T + 1))},
        # every resident weight byte read once per call, over the call's time
        "weights_GBps_over_call": round(weight_bytes / dt / 1e9, 1),
        "tokens_per_expert_max": int(counts.max()),
        "tokens_per_expert_median": float(np.median(counts[counts > 0])),
        "tokens_per_expert_min": int(counts[counts > 0].min()),
        "parity": par,
    }


def run_mtp(args, coli, dev):
    """MTP-verify batches: gs64 scales, 8 tokens per call, router logits with
    Zipf(1.1) popularity (Gumbel top-k), bias 0; K timed calls (125 = 1,000
    tokens) replayed from one graph. Routing of every timed token and the
    outputs of 8 whole calls spread over the run are checked against the
    oracle."""
    import torch
    import oracle
    import synth
    H, I, E, k, T = 6144, 2048, 256, 8, 8
    shape = coli.MoEShape(H, I, E, 1, k, 64, 1.0)
    steps = max(1, args.steps)
    warm = max(1, args.warmup)
    n = steps + warm
    lg_np = synth.zipf_logits(args.seed, 0, 0, n * T, E, s=1.1)
    x_np = synth.activations(args.seed, 0, 0, n * T, H)
    parity = not args.no_parity
    psteps = warm + spread(steps, max(1, args.parity_tokens // T))
    prow = np.concatenate([np.arange(s * T, (s + 1) * T) for s in psteps])
    need = set(np.unique(oracle.route(lg_np[prow], None, k)[0]).tolist()) if parity else set()
    t0 = time.perf_counter()
    arena, table, shared, qx = build_experts(coli, shape, args.seed, dev, oracle_ids=need | {E})
    log(f"gs64 experts ready in {time.perf_counter() - t0:.1f} s")
    lg = torch.from_numpy(lg_np).to(dev)
    x = torch.from_numpy(x_np).to(dev)
    y = torch.empty((n * T, H), dtype=torch.float32, device=dev)
    idx = torch.empty((n * T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((n * T, k), dtype=torch.float32, device=dev)
    ws = coli.workspace(shape, T, coli.PATH_GEMV, dev)
    stream = torch.cuda.Stream()

    def call(i):
        sl = slice(i * T, (i + 1) * T)
        coli.layer_fwd(shape, x[sl], table=table, shared_blob=shared, logits=lg[sl], y=y[sl],
                       idx_out=idx[sl], w_out=wts[sl], path=coli.PATH_GEMV, ws=ws, stream=stream)

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
    ms = time_replays(graph, stream, 1)
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
    par = None
    if parity:
        idx_ref, w_ref = oracle.route(lg_np, None, k)
        experts, sh = oracle_list(qx, shape)
        _, y64, _, _ = oracle.layer(x_np[prow], experts, sh, k, 64, 1.0, logits=lg_np[prow])
        idx_g = idx.cpu().numpy()
        # the union of every timed step against the oracle's
        union_bad = 0
        for s_ in range(warm, n):
            rows = slice(s_ * T, (s_ + 1) * T)
            c, o, p, u, nu = coli.union(idx[rows], E)
            c_r, o_r, p_r, u_r = oracle.union(idx_ref[rows], E)
            ok = (np.array_equal(c.cpu().numpy(), c_r) and np.array_equal(o.cpu().numpy(), o_r)
                  and np.array_equal(p.cpu().numpy(), p_r) and int(nu.cpu()[0]) == len(u_r)
                  and np.array_equal(u.cpu().numpy()[:len(u_r)], u_r))
            union_bad += 0 if ok else 1
        par = {"idx_tokens_checked": n * T,
               "idx_mismatch_tokens": int((idx_g != idx_ref).any(axis=1).sum()),
               "w_mismatch_tokens": int((wts.cpu().numpy() != w_ref).any(axis=1).sum()),
               "union_steps_checked": steps, "union_mismatch_steps": union_bad,
               **check_outputs(y.cpu().numpy()[prow], y64, 1e-3)}
        par["pass"] = bool(par["idx_mismatch_tokens"] == 0 and par["w_mismatch_tokens"] == 0
                           and union_bad == 0 and par["y_pass"])
        log(f"mtp parity: {par}")
    return {
        "metric": "MTP-verify tokens/s (gs64, 8-token batches; weight GB/s vs HBM peak)",
        "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": round(1e3 * elapsed / steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 weights (gs64) x 16-bit block-scaled activations (four signed base-16 "
                 "digit planes per 32-element block), exact int32 block sums, f32 accumulate",
        "data": "synthetic (seeded Philox N(0,0.02) weights, N(0,1) activations, Zipf(1.1) logits)",
        "config": {"workload": "MTP-verify batches of 8 tokens, GLM-5.2-shaped layer, gs64",
                   "hidden": H, "inter": I, "n_routed": E, "top_k": k, "group": 64,
                   "tokens": steps * T, "graph": True},
        "unique_experts_per_token": round(float(uniq.mean()) / T, 3),
        "unique_experts_per_step_mean": round(float(uniq.mean()), 2),
        "unique_experts_per_step_range": [int(uniq.min()), int(uniq.max())],
        "weight_bytes_per_step_mean": round(float((gu_bytes + dn_bytes).mean())),
        "roofline": {"bound": "hbm", "kernel": "gemv_gateup + gemv_down",
                     "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "avg_gateup_us": round(gu_s * 1e6, 2), "avg_down_us": round(dn_s * 1e6, 2)},
        "parity": par,
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
        "dtype": "int4 weights x 16-bit block-scaled activations (four signed base-16 digit planes "
                 "per 32-element block), exact int32 block sums, f32 accumulate",
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
        "roofline": {"bound": "hbm", "kernel": "fp8_wave_kernel (2 launches per expert: gate and up together, then down)",
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


def run_readprobe(args, coli, dev):
    """Read-only streaming kernels (coli_read_probe) over the byte counts of
    the decode GEMVs, in their access patterns and in plain contiguous chunks.
    Each pattern: a graph of launches over N_ROTATE copies of its buffer (so
    the MALL holds none of it between reads), replayed `reps` times, HIP
    events on the stream; median replay / launches."""
    import torch
    gu_bytes = 9 * 2 * 2048 * 3072               # int4 gate and up rows of 9 experts
    dn_bytes = 9 * 6144 * 1024                   # int4 down rows of 9 experts
    blob_bytes = 9 * 18915328                    # 9 whole per-row blobs
    cases = [
        ("gateup_rows", "rows of 3072 B, 3 waves per row, 32 rows per workgroup (decode gate/up)",
         gu_bytes, 1, 3072, 32),
        ("gateup_rows16", "rows of 3072 B, 3 waves per row, 16 rows per workgroup",
         gu_bytes, 1, 3072, 16),
        ("gateup_chunks", "contiguous 96 KB per workgroup", gu_bytes, 0, 98304, 0),
        ("down_rows", "rows of 1024 B, 4 waves x 8 rows per workgroup (decode down)",
         dn_bytes, 1, 1024, 32),
        ("down_chunks", "contiguous 32 KB per workgroup", dn_bytes, 0, 32768, 0),
        ("blobs_chunks", "9 whole blobs, contiguous 96 KB per workgroup", blob_bytes - blob_bytes % 98304 + 98304, 0, 98304, 0),
    ]
    stream = torch.cuda.Stream()
    reps = max(3, min(args.steps, 20))
    out = {}
    for name, what, nbytes, pattern, rb, rpw in cases:
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(i) for i in range(N_ROTATE)]
        sink = torch.empty(1 << 20, dtype=torch.int32, device=dev)
        with torch.cuda.stream(stream):
            for b in bufs:
                coli.read_probe(b, pattern, rb, rpw, sink, stream=stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        launches = 4 * N_ROTATE
        with torch.cuda.graph(g, stream=stream):
            for i in range(launches):
                coli.read_probe(bufs[i % N_ROTATE], pattern, rb, rpw, sink, stream=stream)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ms = time_replays(g, stream, reps)
        us = float(np.median(ms)) * 1e3 / launches
        out[name] = {"pattern": what, "bytes": nbytes, "us_per_launch": round(us, 3),
                     "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "frac_of_8TBps": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
        log(f"readprobe {name}: {us:.2f} us, {out[name]['GBps']} GB/s")
        del g, bufs
        torch.cuda.empty_cache()
    best = max(v["GBps"] for v in out.values())
    return {"metric": "HBM read ceiling by access pattern (read-only streaming kernels)",
            "value": best, "unit": "GB/s", "n_gpus": 1, "steps": reps, "higher_is_better": True,
            "data": "synthetic (constant bytes)", "mall": f"cold ({N_ROTATE} rotating copies)",
            "patterns": out}


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
        args.steps = {"stream": 512, "mtp": 125, "decode": 10}.get(args.workload, 10)
    if args.gpus != 1:
        print(json.dumps({"error": "one-GPU benchmark: the layer runs on a single GPU here (how it "
                                   "would shard is described, not run); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import int4_routed_expert_sigmoid_amd as coli

    coli.lib()                              # fails loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    if args.workload == "decode":
        line = run_decode(args, coli, dev)
    elif args.workload == "copy":
        line = run_copy(args, dev)
    elif args.workload == "prefill":
        shape = coli.MoEShape(6144, 2048, 256, 1, 8, args.group, 1.0)
        parity = not args.no_parity
        need = set()
        if parity:
            import oracle
            import synth
            lgp = synth.zipf_logits(args.seed, 1, 0, 2048, 256, s=1.1, mix=args.prefill_mix)
            need = set(np.unique(oracle.route(lgp[spread(2048, args.parity_tokens)], None, 8)[0]).tolist())
        arena, table, shared, qx = build_experts(coli, shape, args.seed, dev,
                                                 oracle_ids=need | {256} if parity else ())
        line = run_prefill(coli, shape, table, shared, args.seed, dev,
                           calls=max(1, min(args.steps, 50)), warmup=max(1, args.warmup),
                           qx=qx if parity else None, parity_tokens=args.parity_tokens,
                           mix=args.prefill_mix)
        line = {"metric": "prefill TFLOP/s (2048 tokens, bf16 MFMA)", "value": line["tflops_layer"],
                "unit": "TFLOP/s", "n_gpus": 1,
                "dtype": "int4 weights (exact bf16 q + 136) x bf16 activations, f32 accumulate",
                "steps": max(1, min(args.steps, 50)),
                "warmup": max(1, args.warmup), **line}
    elif args.workload == "mtp":
        line = run_mtp(args, coli, dev)
    elif args.workload == "convert":
        line = run_convert(args, coli, dev)
    elif args.workload == "readprobe":
        line = run_readprobe(args, coli, dev)
    else:
        line = run_stream(args, coli, dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
