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
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--graph", type=int, default=1, help="replay the timed tokens from a HIP graph")
    ap.add_argument("--cpu-sample", type=int, default=8, help="tokens of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 2048-token prefill line")
    return ap.parse_args()


def build_experts(coli, shape, seed, dev, keep_host=()):
    """All routed + shared experts quantised on the GPU from seeded f32 weights.
    Returns (arena, table, shared_blob, host f32 copies of `keep_host`)."""
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
        synth.expert_matrix(seed, 0, e, synth.MAT_GATE, I, H, out=g_h.numpy())
        synth.expert_matrix(seed, 0, e, synth.MAT_UP, I, H, out=u_h.numpy())
        synth.expert_matrix(seed, 0, e, synth.MAT_DOWN, H, I, out=d_h.numpy())
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


def cpu_baseline_decode(shape, seed, wr, b, x_all, sample, kept):
    """The oracle's whole layer on `sample` tokens of the same workload."""
    import oracle
    H, I, E, k = shape.hidden, shape.inter, shape.n_routed, shape.top_k
    z = np.zeros((I, H), np.float32)
    zero = oracle.QExpert.quantize(z, z, np.zeros((H, I), np.float32), 0)
    experts = [zero] * E
    for e, (g, u, d) in kept.items():
        if e < E:
            experts[e] = oracle.QExpert.quantize(g, u, d, 0)
    shared = oracle.QExpert.quantize(*kept[E], 0)
    x = np.ascontiguousarray(x_all[:sample])
    t0 = time.perf_counter()
    oracle.layer(x, experts, shared, k, 0, 1.0, wr=wr, bias=b)
    dt = time.perf_counter() - t0
    return {"value": sample / dt, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {sample} tokens of the decode workload, whole layer (router logits, "
                      f"route, union, 9 expert FFNs, combine), scalar C, f64 accumulation, "
                      f"OpenMP over output rows; {dt:.2f} s"}


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
    return {
        "workload": "prefill, 2048 tokens, Zipf(1.1) + 10% uniform routing, same layer",
        "tokens_per_s": round(T / dt, 1),
        "ms_per_call": round(dt * 1e3, 4),
        "tflops_layer": round((flops_gu + flops_dn) / dt / 1e12, 2),
        "gemm_gateup_us": round(gu_s * 1e6, 2),
        "gemm_down_us": round(dn_s * 1e6, 2),
        "gemm_tflops": round((flops_gu + flops_dn) / (gu_s + dn_s) / 1e12, 2) if n_gu else None,
        "gemm_frac_of_bf16_peak": round((flops_gu + flops_dn) / (gu_s + dn_s) / 1e12 / BF16_PEAK_TFLOPS, 4) if n_gu else None,
        "algorithmic_tflop": round((flops_gu + flops_dn) / 1e12, 4),
        "experts_used": int((counts > 0).sum()),
        "tokens_per_expert_max": int(counts.max()),
        "tokens_per_expert_median": float(np.median(counts[counts > 0])),
        "tokens_per_expert_min": int(counts[counts > 0].min()),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import synth
    import int4_routed_expert_sigmoid_amd as coli
    import oracle

    dev = torch.device("cuda:0")
    H, I, E, k = 6144, 2048, 256, 8
    shape = coli.MoEShape(H, I, E, 1, k, 0, 1.0)
    seed = args.seed
    n_tok = args.warmup + args.steps
    log(f"decode workload: {n_tok} tokens, H={H} I={I} E={E}+1 k={k}")

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
    ws = coli.workspace(shape, 1, coli.PATH_GEMV, dev)

    def token(t):
        coli.layer_fwd(shape, x_d[t:t + 1], table=table, shared_blob=shared, router_w=wr_d,
                       bias=b_d, y=y_d[t:t + 1], path=coli.PATH_GEMV, ws=ws)

    stream = torch.cuda.Stream()
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
    # recorded around each GEMV kernel on the stream it runs on (HIP cannot
    # time events recorded inside a captured graph)
    coli.profile_enable(2 * args.steps + 16)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for t in range(args.warmup, n_tok):
            token(t)
    torch.cuda.synchronize()
    elapsed_eager = time.perf_counter() - t0
    n_gu, ms_gu = coli.profile_summary("gemv_gateup")
    n_dn, ms_dn = coli.profile_summary("gemv_down")
    coli.profile_enable(0)
    elapsed = elapsed_graph if graph is not None else elapsed_eager

    # algorithmic bytes per token: 9 blobs (8 routed + shared)
    gu_bytes = 9 * (2 * I * (H // 2) + 2 * I * 4)
    dn_bytes = 9 * (H * (I // 2) + H * 4)
    gu_avg_s = ms_gu / max(1, n_gu) / 1e3
    dn_avg_s = ms_dn / max(1, n_dn) / 1e3
    gu_gbps = gu_bytes / gu_avg_s / 1e9 if n_gu else None
    dn_gbps = dn_bytes / dn_avg_s / 1e9 if n_dn else None
    gemv_gbps = (gu_bytes + dn_bytes) / (gu_avg_s + dn_avg_s) / 1e9 if n_gu and n_dn else None
    tok_s = args.steps / elapsed

    prefill = None
    if not args.no_prefill:
        log("prefill: 2048 tokens through the same layer (bf16 MFMA)")
        prefill = run_prefill(coli, shape, table, shared, seed, dev)

    cpu = None
    if sample:
        cpu = cpu_baseline_decode(shape, seed, wr, b, x_all, sample, kept)

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
        "dtype": "int4 weights x f32 activations (exact int32 nibble products), f32 accumulate",
        "data": "synthetic (seeded Philox N(0,0.02) weights, N(0,1) activations, f32 router)",
        "config": {"workload": "GLM-5.2-shaped MoE layer, batch-1 decode", "hidden": H,
                   "inter": I, "n_routed": E, "n_shared": 1, "top_k": k, "group": 0,
                   "tokens": args.steps, "graph": bool(args.graph),
                   "eager_tokens_per_s": round(args.steps / elapsed_eager, 2)},
        "roofline": {"bound": "hbm", "kernel": "gemv_gateup",
                     "achieved": round(gu_gbps, 1) if gu_gbps else None,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gu_gbps / HBM_PEAK_GBPS, 4) if gu_gbps else None,
                     "traffic": None,
                     "bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_avg_s * 1e6, 3),
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
