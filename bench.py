#!/usr/bin/env python3
"""Benchmark of one draft-tree verification step on one MI355X.

A step is the whole hot path over one batch: ancestor-mask build,
tree-masked split-KV GQA attention (one layer) and greedy acceptance, at the
headline workload (8 sequences of which 6 live, 28/4 heads, head_dim 128,
bf16, contexts 4096-8192, 32-node trees, vocabulary 152064). Inputs are
seeded synthetic tensors resident in HBM before timing starts. The timed
loop rotates over several copies of the inputs so that the 256 MB Infinity
Cache cannot serve a step from the previous one (cold timing).

Prints one JSON line. ``value`` is verified draft nodes per second for the
whole step; ``roofline`` reports the attention call against whichever of
its two bounds binds (matrix-core flops at 2.5 PFLOP/s, or algorithmic HBM
bytes at 8 TB/s), from HIP events recorded on the stream the kernels run
on; ``cpu_baseline`` times the float64 oracle on a bounded sample of the
same workload on the host.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "verified draft nodes/sec + achieved HBM GB/s (B=8, 8k ctx, N=32 tree)"
# Cold timing: the rotated input copies together exceed three times the
# 256 MiB Infinity Cache, so no call finds its inputs left there by the
# previous ones.
MIN_SETS = 10
COLD_MIB = 768
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_traffic.json")
ATTN_SRC = os.path.join(ROOT, "tree_attention_draft_tv_amd", "csrc", "tv_attention.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200,
                    help="timed steps (a step is ~85 us: fewer leave the wall clock to jitter)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="C3", help="workload (C1..C5); C3 is the headline")
    ap.add_argument("--sets", type=int, default=0,
                    help="input copies rotated for cold timing (0: at least %d and at least "
                         "%d MiB of inputs, three times the Infinity Cache)" % (MIN_SETS,
                                                                                  COLD_MIB))
    ap.add_argument("--chunk", type=int, default=0, help="attention chunk_keys (0 = auto)")
    ap.add_argument("--parts", type=int, default=3,
                    help="probability_parts (3: fp32-faithful probabilities, the page's "
                         "setting; 1: the lossy fast mode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="target host time of each oracle baseline sample (the step, then "
                         "attention and acceptance each on one thread and on all cores)")
    ap.add_argument("--no-sampling", action="store_true",
                    help="skip the secondary sampling-acceptance measurement")
    ap.add_argument("--no-projections", action="store_true",
                    help="skip the few-row projection measurement")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the long-context (32768-key) attention measurement")
    ap.add_argument("--no-packed", action="store_true",
                    help="skip the packed-row attention and budget-controller measurement")
    ap.add_argument("--commit-layers", type=int, default=28,
                    help="layers of the KV-commit measurement (0 skips it)")
    ap.add_argument("--graph", type=int, default=0,
                    help="1: replay the steps from a captured HIP graph (the library's calls "
                         "are graph-capturable); 0: launch them one by one")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the streaming-read measurement")
    return ap.parse_args()


def attention_alg_bytes(w):
    """Bytes the attention must move: live committed + tree K and V, live
    queries, fp32 outputs and LSE, and the mask words."""
    elt = 2 if w.dtype == "bf16" else 4
    tot = 0
    for b in range(w.B):
        n = int(w.n_nodes[b])
        if n == 0:
            continue
        L = int(w.ctx_len[b])
        tot += 2 * (L + n) * w.Hkv * w.D * elt        # K and V
        tot += n * w.Hq * w.D * elt                   # Q
        tot += n * w.Hq * w.D * 4 + n * w.Hq * 4      # out + lse
        tot += n * ((w.T + 31) // 32) * 4             # mask
    return tot


def attention_flops(w, parts):
    """Matrix-core flops the attention must issue: per live packed row and
    per key of its sequence (committed or tree), 2 D for Q K^T and 2 D per
    probability part for P V (the parts are separate bf16 products)."""
    tot = 0
    for b in range(w.B):
        n = int(w.n_nodes[b])
        if n:
            tot += (2 + 2 * parts) * w.D * w.G * n * (int(w.ctx_len[b]) + n) * w.Hkv
    return tot


def accept_alg_bytes(w):
    """Inputs of the acceptance read once: every live logits row, and in
    sampling mode the draft row and uniform of every non-root live node,
    plus the small per-node words (parent, token, outputs)."""
    tot = 0
    for b in range(w.B):
        n = int(w.n_nodes[b])
        tot += n * w.V * 4 + n * 8 * 4
        if w.qdraft is not None:
            tot += max(n - 1, 0) * (w.V * 4 + 4)
    return tot


def cold_sets(per_set_bytes, requested=0):
    """Number of input copies to rotate: `requested`, else enough that they
    total COLD_MIB MiB, and at least MIN_SETS."""
    if requested:
        return requested
    return max(MIN_SETS, -(-(COLD_MIB << 20) // max(1, per_set_bytes)))


def kernel_source_hash():
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per attention launch from the committed counter runs, if the
    kernel source is unchanged since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def _oracle_rate(w, seconds, parts):
    """Verified draft nodes per second of the float64 oracle running `parts`
    ("mask", "attention", "accept") one live sequence at a time until about
    `seconds` of host time have passed. Returns (rate, sequences, seconds)."""
    import oracle
    live = [b for b in range(w.B) if w.n_nodes[b] > 0]
    nodes = seqs = i = 0
    t0 = time.perf_counter()
    while True:
        b = live[i % len(live)]
        sl = slice(b, b + 1)
        if "mask" in parts:
            oracle.build_tree_mask(w.parent[sl], w.n_nodes[sl], w.T)
        if "attention" in parts:
            oracle.tree_attention(w.q[sl], w.k[sl], w.v[sl], w.dtype, w.ctx_len[sl],
                                  w.n_nodes[sl], w.parent[sl], w.scale)
        if "accept" in parts:
            if w.mode == "greedy":
                oracle.accept_greedy(w.logits[sl], w.tokens[sl], w.parent[sl], w.n_nodes[sl])
            else:
                oracle.accept_sample(w.logits[sl], w.temperature, w.qdraft[sl], w.u[sl],
                                     w.tokens[sl], w.parent[sl], w.n_nodes[sl])
        nodes += int(w.n_nodes[b]) - 1
        seqs += 1
        i += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return nodes / el, seqs, el


def cpu_baseline(w, seconds):
    """The float64 oracle on the host: the whole step on all cores (the
    reported value), then attention and acceptance apart, each on one thread
    and on all cores. Each sample runs whole live sequences of the workload
    for about `seconds`."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threadpool_limits = None
        threads = os.cpu_count() or 1
    rate, seqs, el = _oracle_rate(w, seconds, ("mask", "attention", "accept"))
    res = {"value": rate, "unit": "verified draft nodes/s", "cores": int(threads),
           "kind": "oracle",
           "sample": "%d sequence(s) of workload %s (mask + float64 attention over all %d KV "
                     "heads + %s acceptance), %.1f s, all cores" % (seqs, w.name, w.Hkv, w.mode,
                                                                   el)}
    for part in ("attention", "accept"):
        entry = {}
        for label, limit in (("one_thread", 1), ("all_cores", None)):
            if limit is not None and threadpool_limits is None:
                continue
            if limit is None:
                r, n_s, e = _oracle_rate(w, seconds / 2, (part,))
                cores = threads
            else:
                with threadpool_limits(limits=limit):
                    r, n_s, e = _oracle_rate(w, seconds / 2, (part,))
                cores = limit
            entry[label] = {"value": round(r, 2), "unit": "verified draft nodes/s",
                            "cores": int(cores), "sample": "%d sequence(s), %.1f s" % (n_s, e)}
        res["attention" if part == "attention" else "acceptance"] = entry
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import tree_attention_draft_tv_amd as tv
    from workloads import make_config

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    tv.load()

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return

    w = make_config(args.config)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32))

    host = {
        "q": bf(w.q) if w.dtype == "bf16" else torch.from_numpy(w.q),
        "k": bf(w.k) if w.dtype == "bf16" else torch.from_numpy(w.k),
        "v": bf(w.v) if w.dtype == "bf16" else torch.from_numpy(w.v),
        "ctx": i32(w.ctx_len), "n": i32(w.n_nodes), "parent": i32(w.parent),
        "tokens": i32(w.tokens), "logits": torch.from_numpy(w.logits),
    }
    if w.mode == "sample":
        host["qd"] = torch.from_numpy(w.qdraft)
        host["u"] = torch.from_numpy(w.u)
    per_set = sum(t.numel() * t.element_size() for t in host.values())
    sets = [{k: t.to(dev) for k, t in host.items()} for _ in range(cold_sets(per_set, args.sets))]
    B, T = w.B, w.T
    W = (T + 31) // 32
    bufs = []
    for _ in sets:
        bufs.append({
            "mask": (torch.empty((B, T, W), dtype=torch.int32, device=dev),
                     torch.empty((B, T), dtype=torch.int32, device=dev),
                     torch.empty((B,), dtype=torch.int32, device=dev)),
            "out": torch.empty((B, T, w.Hq, w.D), dtype=torch.float32, device=dev),
            "lse": torch.empty((B, T, w.Hq), dtype=torch.float32, device=dev),
            "ast": torch.empty((B,), dtype=torch.int32, device=dev),
        })
    ws_attn = torch.empty(max(1, tv.attention_workspace_size(B, T, w.Hq, w.Hkv, w.D, w.max_ctx,
                                                               args.chunk)),
                          dtype=torch.uint8, device=dev)
    mode = 0 if w.mode == "greedy" else 1
    ws_acc = torch.empty(tv.accept_workspace_size(B, T, w.V, mode), dtype=torch.uint8, device=dev)
    acc_out = (torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B, T), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B, T), dtype=torch.uint8, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    dec = torch.empty((B, T), dtype=torch.int8, device=dev)

    def do_mask(i):
        s = sets[i % len(sets)]
        bb = bufs[i % len(bufs)]
        return tv.build_tree_mask(s["parent"], s["n"], out=bb["mask"])[0]

    def do_attention(i):
        s = sets[i % len(sets)]
        bb = bufs[i % len(bufs)]
        tv.tree_attention(s["q"], s["k"], s["v"], s["ctx"], s["n"], bb["mask"][0], w.max_ctx,
                          scale=float(w.scale), probability_parts=args.parts,
                          chunk_keys=args.chunk, out=bb["out"], lse=bb["lse"],
                          row_status=bb["ast"], workspace=ws_attn)

    def do_accept(i):
        s = sets[i % len(sets)]
        if mode == 0:
            tv.accept_greedy(s["logits"], s["tokens"], s["parent"], s["n"], outputs=acc_out,
                             workspace=ws_acc)
        else:
            tv.accept_sample(s["logits"], float(w.temperature), s["qd"], s["u"], s["tokens"],
                             s["parent"], s["n"], outputs=acc_out[:4] + (dec, acc_out[4]),
                             workspace=ws_acc)

    def step(i):
        do_mask(i)
        do_attention(i)
        do_accept(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region 1: whole steps, wall clock between two synchronisations.
    # With --graph 1 one graph holds one step per input copy and is replayed.
    nsets = len(sets)
    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(nsets):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(nsets):
                step(i)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
    steps = args.steps
    if graph is not None:
        steps = max(nsets, (args.steps + nsets - 1) // nsets * nsets)
    t0 = time.perf_counter()
    if graph is not None:
        for _ in range(steps // nsets):
            graph.replay()
    else:
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Timed region 2: each call of the step on its own, `reps` calls back to
    # back between two HIP events recorded on the stream the kernels are
    # launched on (torch's current stream, which the binding passes to the
    # library); the average includes the launch gaps inside a call.
    reps = max(20, min(args.steps, 100))
    timed = lambda fn: time_calls(torch, fn, reps)

    t_mask = timed(do_mask)
    # Attention: 10 timed replays of 20 calls (200 calls after the warm-up),
    # reported as the mean and the spread of the replay averages.
    t_attn, attn_rounds = time_calls(torch, do_attention, 20, rounds=10)
    t_acc = timed(do_accept)
    # The lossy fast mode (one bf16 probability part, 16-bit partials) on the
    # same inputs, as a labelled secondary figure.
    t_fast = None
    if args.parts != 1:
        def do_attention_fast(i):
            s = sets[i % len(sets)]
            bb = bufs[i % len(bufs)]
            tv.tree_attention(s["q"], s["k"], s["v"], s["ctx"], s["n"], bb["mask"][0], w.max_ctx,
                              scale=float(w.scale), probability_parts=1,
                              chunk_keys=args.chunk, out=bb["out"], lse=bb["lse"],
                              row_status=bb["ast"], workspace=ws_attn)
        t_fast = time_calls(torch, do_attention_fast, 20, rounds=5)[0]

    ms_per_step = wall / steps * 1e3
    nodes = w.draft_nodes
    value = nodes / (wall / steps)
    a_bytes = attention_alg_bytes(w)
    a_flops = attention_flops(w, args.parts)
    acc_bytes = accept_alg_bytes(w)
    achieved = a_bytes / t_attn / 1e9
    # The roofline is the bound that binds: HBM bytes at 8 TB/s or bf16
    # matrix-core flops at 2.5 PFLOP/s (three probability parts triple the
    # P V products, which makes the call MFMA-bound at C3).
    t_hbm, t_mfma = a_bytes / (PEAK_HBM_GBS * 1e9), a_flops / (PEAK_BF16_TFLOPS * 1e12)
    mfma_bound = t_mfma > t_hbm
    achieved_tf = a_flops / t_attn / 1e12
    traffic = measured_traffic()
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "verified draft nodes/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; cold: %d rotating input copies, %.0f MiB)%s" % (
            len(sets), len(sets) * per_set / 2 ** 20,
            "; steps replayed from a HIP graph" if graph is not None else ""),
        "config": {
            "workload": "%s: B=%d (%d live), Hq/Hkv=%d/%d, D=%d, ctx %d..%d, N=%d draft nodes "
                        "(T=%d), V=%d, %s acceptance" % (
                            w.name, w.B, w.live_rows, w.Hq, w.Hkv, w.D, int(w.ctx_len.min()),
                            int(w.ctx_len.max()), w.T - 1, w.T, w.V, w.mode),
            "draft_nodes_per_step": nodes,
            "chunk_keys": args.chunk if args.chunk else "balanced on the device",
            "probability_parts": args.parts,
        },
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "kernel": "tv_tree_attention (split + combine)",
            "achieved": round(achieved_tf if mfma_bound else achieved, 1),
            "peak": PEAK_BF16_TFLOPS if mfma_bound else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round(achieved_tf / PEAK_BF16_TFLOPS if mfma_bound
                          else achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": a_bytes,
            "alg_flops_per_launch": a_flops,
            "time_at_peak_us": {"hbm": round(t_hbm * 1e6, 3), "mfma": round(t_mfma * 1e6, 3)},
            "hbm_GBps": round(achieved, 1),
            "hbm_frac": round(achieved / PEAK_HBM_GBS, 4),
            "mfma_TFLOPs": round(achieved_tf, 1),
            "mfma_frac": round(achieved_tf / PEAK_BF16_TFLOPS, 4),
            "avg_launch_us": round(t_attn * 1e6, 3),
            "launch_us_p10_p50_p90": [round(float(np.percentile(attn_rounds, q)) * 1e6, 3)
                                      for q in (10, 50, 90)],
        },
        "kernels": {
            "mask_us": round(t_mask * 1e6, 3),
            "attention_us": round(t_attn * 1e6, 3),
            "attention_GBps": round(achieved, 1),
            "attention_TFLOPs": round(a_flops / t_attn / 1e12, 2),
            "accept_us": round(t_acc * 1e6, 3),
            "accept_GBps": round(acc_bytes / t_acc / 1e9, 1),
            "accept_alg_bytes": acc_bytes,
            "nodes_per_s_attention_only": round(nodes / t_attn, 1),
        },
    }
    if t_fast is not None:
        res["fast_mode_attention"] = {
            "probability_parts": 1, "note": "lossy: bf16 probabilities, 16-bit split partials",
            "attention_us": round(t_fast * 1e6, 3),
            "GBps": round(a_bytes / t_fast / 1e9, 1),
            "hbm_frac": round(a_bytes / t_fast / 1e9 / PEAK_HBM_GBS, 4)}

    if not args.no_sampling and w.mode == "greedy":
        res["sampling"] = sampling_secondary(tv, torch, dev, args)
    if not args.no_projections and w.dtype == "bf16":
        res["projections"] = projections_secondary(tv, torch, dev, w, args)
    if args.commit_layers > 0 and w.mode == "greedy":
        res["kv_commit"] = commit_secondary(tv, torch, dev, w, sets[0], acc_out, args)
    if not args.no_packed:
        res["packed_rows"] = packed_secondary(tv, torch, dev, w, sets, bufs, ws_attn, acc_out,
                                              t_attn, args)
    if not args.no_long_context and args.config == "C3":
        res["long_context"] = long_context_secondary(tv, torch, dev, args)

    if not args.no_read_ceiling:
        ceil = read_ceiling(tv, torch, dev)
        res["roofline"]["measured_read_ceiling_GBps"] = ceil["GBps"]
        res["roofline"]["hbm_frac_of_measured_ceiling"] = round(achieved / ceil["GBps"], 4)
        res["read_ceiling"] = ceil
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def projections_secondary(tv, torch, dev, w, args):
    """Batch-invariant few-row projections of the B*T verification rows:
    the fused Q/K/V projection (hidden 3584 = 28 x 128 -> 28 + 4 + 4 heads of
    128) and gate/up with the rounded SwiGLU (intermediate 18944), the sizes
    of a Qwen2-7B-class decoder layer; random bf16 weights. torch.matmul
    (hipBLASLt) on the same shapes is timed beside them as context. Warm."""
    M, K = w.B * w.T, w.Hq * w.D
    n_qkv, n_ffn = (w.Hq + 2 * w.Hkv) * w.D, 18944
    g = torch.Generator(device=dev).manual_seed(11)
    x = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
    wq = (torch.randn((n_qkv, K), generator=g, device=dev) / K ** 0.5).to(torch.bfloat16)
    wg = (torch.randn((n_ffn, K), generator=g, device=dev) / K ** 0.5).to(torch.bfloat16)
    wu = (torch.randn((n_ffn, K), generator=g, device=dev) / K ** 0.5).to(torch.bfloat16)
    yq = torch.empty((M, n_qkv), dtype=torch.bfloat16, device=dev)
    yf = torch.empty((M, n_ffn), dtype=torch.bfloat16, device=dev)
    reps = max(20, min(args.steps, 100))
    t_qkv = time_calls(torch, lambda i: tv.linear_rows(x, wq, out=yq), reps)
    t_ffn = time_calls(torch, lambda i: tv.linear_swiglu_rows(x, wg, wu, out=yf), reps)
    t_qkv_ref = time_calls(torch, lambda i: torch.matmul(x, wq.t()), reps)
    t_ffn_ref = time_calls(torch, lambda i: torch.nn.functional.silu(torch.matmul(x, wg.t())) *
                           torch.matmul(x, wu.t()), reps)
    b_qkv = 2 * (n_qkv * K + M * K + M * n_qkv)
    b_ffn = 2 * (2 * n_ffn * K + M * K + M * n_ffn)
    return {"rows": M, "hidden": K,
            "qkv": {"N": n_qkv, "us": round(t_qkv * 1e6, 3), "alg_bytes": b_qkv,
                    "GBps": round(b_qkv / t_qkv / 1e9, 1),
                    "torch_matmul_us": round(t_qkv_ref * 1e6, 3)},
            "gate_up_swiglu": {"N": n_ffn, "us": round(t_ffn * 1e6, 3), "alg_bytes": b_ffn,
                               "GBps": round(b_ffn / t_ffn / 1e9, 1),
                               "torch_matmul_silu_mul_us": round(t_ffn_ref * 1e6, 3)}}


def time_calls(torch, fn, reps, rounds=1):
    """Average GPU time of fn(i) over `reps` back-to-back calls. The calls are
    captured once in a HIP graph and replayed between two events, so that
    the host's launch path (~10 us per call through the binding) does not
    pace kernels shorter than it; eager launches if capture fails. With
    rounds > 1 the replay is timed that many times and (mean, [per-round
    averages]) is returned."""
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    graph = torch.cuda.CUDAGraph()
    try:
        with torch.cuda.graph(graph):
            for i in range(reps):
                fn(i)
        graph.replay()
        torch.cuda.synchronize()
    except RuntimeError:
        graph = None
        torch.cuda.synchronize()
    per_round = []
    for _ in range(rounds):
        e0.record()
        if graph is not None:
            graph.replay()
        else:
            for i in range(reps):
                fn(i)
        e1.record()
        torch.cuda.synchronize()
        per_round.append(e0.elapsed_time(e1) * 1e-3 / reps)
    if rounds == 1:
        return per_round[0]
    return sum(per_round) / rounds, per_round


def commit_secondary(tv, torch, dev, w, s, acc_out, args):
    """Accepted-path KV commit after the greedy acceptance of the same step,
    into `layers` bf16 caches [layers, B, Hkv, capacity, D] (contents are
    moved bit for bit, so they need no values); warm."""
    layers = args.commit_layers
    tv.accept_greedy(s["logits"], s["tokens"], s["parent"], s["n"], outputs=acc_out)
    acc_len, path = acc_out[0], acc_out[1]
    shape = (layers, w.B, w.Hkv, w.kv_capacity, w.D)
    k = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    v = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    new_ctx = torch.empty((w.B,), dtype=torch.int32, device=dev)
    st = torch.empty((w.B,), dtype=torch.int32, device=dev)

    def call(i):
        tv.commit_accepted_kv(k, v, s["ctx"], s["n"], acc_len, path, new_ctx_len=new_ctx,
                              row_status=st)

    t = time_calls(torch, call, max(20, min(args.steps, 100)))
    moved = int(acc_len.sum().item())
    by = moved * w.Hkv * w.D * 2 * 2 * 2 * layers  # K and V rows, read + write, bf16
    return {"workload": "C3 greedy acceptance, %d layers" % layers, "accepted_nodes": moved,
            "commit_us": round(t * 1e6, 3), "alg_bytes": by, "GBps": round(by / t / 1e9, 1)}


def packed_secondary(tv, torch, dev, w, sets, bufs, ws_attn, acc_out, t_padded, args):
    """The same attention over packed query rows (live rows back to back, one
    spare row between sequences), cold like the headline call, and the
    device-side budget controller fed by the step's acceptance."""
    n = w.n_nodes.astype(np.int64)
    start = np.zeros(w.B, np.int32)
    pos = 0
    for b in range(w.B):
        start[b] = pos
        pos += int(n[b]) + 1
    rows = pos
    start_d = torch.from_numpy(start).to(dev)
    packed = []
    for s in sets:
        q = torch.empty((rows, w.Hq, w.D), dtype=s["q"].dtype, device=dev)
        for b in range(w.B):
            q[int(start[b]):int(start[b]) + int(n[b])] = s["q"][b, :int(n[b])]
        packed.append(q)
    out = torch.empty((rows, w.Hq, w.D), dtype=torch.float32, device=dev)
    lse = torch.empty((rows, w.Hq), dtype=torch.float32, device=dev)
    st = torch.empty((w.B,), dtype=torch.int32, device=dev)

    def call(i):
        s = sets[i % len(sets)]
        tv.tree_attention_packed(packed[i % len(sets)], s["k"], s["v"], s["ctx"], s["n"],
                                 bufs[i % len(bufs)]["mask"][0], start_d, w.max_ctx,
                                 scale=float(w.scale), probability_parts=args.parts,
                                 chunk_keys=args.chunk, out=out, lse=lse, row_status=st,
                                 workspace=ws_attn)

    t = time_calls(torch, call, max(20, min(args.steps, 100)))
    ema = torch.full((w.B,), 0.5, dtype=torch.float32, device=dev)
    bud = torch.full((w.B,), w.T - 1, dtype=torch.int32, device=dev)
    rs = torch.empty((w.B,), dtype=torch.int32, device=dev)
    rt = torch.empty((1,), dtype=torch.int32, device=dev)

    def ctl(i):
        tv.adapt_tree_budget(acc_out[0], sets[0]["n"], ema, bud, 0.5, 0.25, 2, w.T - 1,
                             row_start=rs, rows_total=rt)

    tc = time_calls(torch, ctl, max(20, min(args.steps, 100)))
    return {"rows": rows, "padded_rows": w.B * w.T, "attention_us": round(t * 1e6, 3),
            "padded_attention_us": round(t_padded * 1e6, 3),
            "budget_controller_us": round(tc * 1e6, 3)}


def long_context_secondary(tv, torch, dev, args):
    """Tree attention at the long-context workload (one sequence, 32768
    committed keys, 65-row tree): the compute-heavier shape, reported against
    the bf16 MFMA peak beside its HBM fraction; cold (rotating input copies
    of the query and KV cache)."""
    from workloads import make_config

    w = make_config("C4")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(  # noqa: E731
        torch.bfloat16)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)  # noqa: E731
    host = [bf(w.q), bf(w.k), bf(w.v)]
    per_set = sum(t.numel() * t.element_size() for t in host)
    sets = [[t.to(dev) for t in host] for _ in range(cold_sets(per_set))]
    ctx, n, par = i32(w.ctx_len), i32(w.n_nodes), i32(w.parent)
    mask = tv.build_tree_mask(par, n)[0]
    ws = torch.empty(max(1, tv.attention_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D, w.max_ctx, 0)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.T, w.Hq, w.D), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.T, w.Hq), dtype=torch.float32, device=dev)
    st = torch.empty((w.B,), dtype=torch.int32, device=dev)

    def call(i):
        q, k, v = sets[i % len(sets)]
        tv.tree_attention(q, k, v, ctx, n, mask, w.max_ctx, scale=float(w.scale), out=out,
                          lse=lse, row_status=st, workspace=ws)

    t = time_calls(torch, call, 4 * len(sets))
    by, fl = attention_alg_bytes(w), attention_flops(w, 3)
    return {"workload": "C4: B=1, Hq/Hkv=28/4, D=128, ctx 32768, N=64 draft nodes (T=65)",
            "cold": "%d rotating input copies, %.0f MiB" % (len(sets), len(sets) * per_set / 2 ** 20),
            "attention_us": round(t * 1e6, 3), "alg_bytes": by, "flops": fl,
            "GBps": round(by / t / 1e9, 1), "hbm_frac": round(by / t / 1e9 / PEAK_HBM_GBS, 4),
            "TFLOPs": round(fl / t / 1e12, 1),
            "mfma_frac": round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4)}


def sampling_secondary(tv, torch, dev, args):
    """Sampling acceptance at its own workload (8 sequences, V=32000,
    temperature 0.7): cold (rotating copies of the logits and draft rows),
    timed from graph replays like the other calls."""
    from workloads import make_config

    w = make_config("C5")
    host = [torch.from_numpy(w.logits), torch.from_numpy(w.qdraft)]
    per_set = sum(t.numel() * t.element_size() for t in host)
    sets = [[t.to(dev) for t in host] for _ in range(cold_sets(per_set))]
    u = torch.from_numpy(w.u).to(dev)
    tok = torch.from_numpy(w.tokens).to(dev)
    par = torch.from_numpy(w.parent).to(dev)
    n = torch.from_numpy(w.n_nodes).to(dev)
    ws = torch.empty(tv.accept_workspace_size(w.B, w.T, w.V, 1), dtype=torch.uint8, device=dev)
    outs = tv.accept_sample(sets[0][0], float(w.temperature), sets[0][1], u, tok, par, n,
                            workspace=ws)

    def call(i):
        lg, qd = sets[i % len(sets)]
        tv.accept_sample(lg, float(w.temperature), qd, u, tok, par, n, outputs=outs, workspace=ws)

    t = time_calls(torch, call, 4 * len(sets))
    by = accept_alg_bytes(w)
    return {"workload": "C5: B=8, V=32000, N=32, temperature 0.7",
            "cold": "%d rotating input copies, %.0f MiB" % (len(sets), len(sets) * per_set / 2 ** 20),
            "accept_us": round(t * 1e6, 3), "alg_bytes": by, "GBps": round(by / t / 1e9, 1),
            "hbm_frac": round(by / t / 1e9 / PEAK_HBM_GBS, 4)}


def read_ceiling(tv, torch, dev):
    """The chip's streaming-read rate: one read of a 4 GiB buffer (coalesced
    16-byte non-temporal loads), timed over graph replays."""
    nbytes = 4 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(7)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    t = time_calls(torch, lambda i: tv.read_probe(buf, sink), 10)
    del buf
    return {"bytes": nbytes, "us": round(t * 1e6, 1), "GBps": round(nbytes / t / 1e9, 1)}


if __name__ == "__main__":
    main()
