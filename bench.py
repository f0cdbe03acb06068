"""Benchmark of the DFlash2 block-drafter hot path on one MI355X.

A step is one draft_block call: the block of G rows of each of B requests through the
five layers, the head, top-k, score_edges and the greedy walk.  Inputs and weights are
synthetic and resident in HBM before the timed region; the context K/V is materialised
once before it (it runs per prefill/commit, not per draft).

Prints one JSON line with the throughput (drafted block tokens/s = B*G / step time), a
per-kernel-class breakdown, the roofline of the dominant kernel (HIP events around its
launches on the launch stream during the timed region), the HBM fraction of the grouped
conv and of the candidate walk, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="full", choices=["full", "long", "tiny", "conv", "selector"],
                   help="full/long/tiny: draft_block; conv, selector: the grouped-conv and "
                        "candidate-selector microbenchmarks")
    p.add_argument("--weights", default="bf16", choices=["bf16", "q4"],
                   help="layer projection weights: bf16, or 4-bit affine (groups of 64); the q4 line "
                        "reports no cpu_baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="full workload: skip the embedded conv, selector and long-workload measurements")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain 1 GiB copy (counter calibration) and exit")
    return p.parse_args()


def pmc_traffic(kernel_class: str, workload: str, weights: str = "bf16"):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were taken
    on the current kernel sources with the same (bf16) weights (null otherwise)."""
    if weights != "bf16":
        return None
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel_class}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "dflash2_block_drafter_amd", "csrc", rec.get("source", ""))
    if not os.path.exists(src):
        return None
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if digest != rec.get("source_sha256"):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.workload in ("conv", "selector"):
        rec = (bench_conv if args.workload == "conv" else bench_selector)(args.steps, args.warmup)
        print(json.dumps(rec), flush=True)
        return

    from dflash2_block_drafter_amd import configs
    w = configs.WORKLOADS[args.workload]
    out = bench_draft(w, args.steps, args.warmup, args.weights, cpu=not args.no_cpu_baseline and args.weights == "bf16")
    if args.workload == "full" and args.weights == "bf16" and not args.no_extras:
        # The metric's second half, "conv+walk % HBM peak", as the grouped-conv microbenchmark
        # (T = 1024 rows) and the candidate-selector chain (B = 32) measure it, each from cold
        # HBM; and the long-context workload (B = 64, L = 8192), where the projections are
        # bound by the matrix cores.
        print("# conv microbenchmark", file=sys.stderr, flush=True)
        out["conv_cfg2"] = _embedded(bench_conv(max(args.steps, 48), args.warmup))
        print("# selector microbenchmark", file=sys.stderr, flush=True)
        out["walk_cfg3"] = _embedded(bench_selector(max(args.steps, 40), args.warmup))
        print("# long workload", file=sys.stderr, flush=True)
        out["long"] = _embedded(bench_draft(configs.LONG, 10, 3, "bf16", cpu=False,
                                            classes=["gemm_head", "gemm_gateup", "attention"]))
    print(json.dumps(out), flush=True)


def _embedded(rec: dict) -> dict:
    """A sub-benchmark's record as embedded in the headline line (without the headline keys)."""
    drop = {"metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data", "cpu_baseline"}
    return {k: v for k, v in rec.items() if k not in drop}


def bench_draft(w, steps: int, warmup: int, weight_kind: str = "bf16", cpu: bool = True, classes=None) -> dict:
    """draft_block on workload w: `warmup` untimed steps, a per-kernel-class breakdown (one step
    per class, that class's launches bracketed by HIP events on the launch stream), then
    `steps` timed steps with the dominant class bracketed the same way (its roofline)."""
    import torch

    from dflash2_block_drafter_amd import binding as B_
    from dflash2_block_drafter_amd import synth
    from dflash2_block_drafter_amd.drafter import Drafter

    d = w.dims
    dev = "cuda"
    torch.cuda.set_device(0)
    t0 = time.time()
    weights = synth.drafter_weights(w, device=dev)
    q4 = synth.drafter_q4_weights(w, device=dev) if weight_kind == "q4" else None
    if q4 is not None:
        for name in q4:
            del weights[name + ".weight"]
    tgt = synth.target_inputs(w, device=dev, with_taps=not w.kv_given)
    dr = Drafter(d, weights, q4_weights=q4)
    del q4
    Bq, G, L = w.batch, d.block_size, w.ctx_len
    if w.kv_given:
        K, V = [], []
        for i in range(d.layers):
            k, v = synth.given_kv(w, i, device=dev)
            K.append(k)
            V.append(v)
        ctx_ms = None
    else:
        K, V = dr.alloc_kv(Bq, L)
        dr.materialize(tgt["taps"], K, V)          # warm call
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        dr.materialize(tgt["taps"], K, V)
        e.record()
        torch.cuda.synchronize()
        ctx_ms = s.elapsed_time(e)
        del tgt["taps"]
    print(f"# {w.name}: inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    ws = dr.workspace(Bq, G, L)
    tokens = torch.empty((Bq, G - 1), dtype=torch.int32, device=dev)
    # the target's head is bound once (copied to the tile-contiguous layout), as a serving
    # loop binds its target before drafting; every step still streams all of it
    dr.bind_target(tgt["lm_head"])

    def step():
        dr.draft(tgt["embeds"], tgt["anchors"], K, V, L, tgt["ctx_len"], tgt["pos0"], tgt["lm_head"],
                 tokens=tokens, ws=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # per-kernel-class breakdown: one step per class with that class bracketed by events
    # (each bracket adds the event's own cost, so short kernels read long here; the kernel
    # trace in profiles/ has their true durations)
    breakdown = {}
    for k in (classes or B_.KERNEL_CLASSES):
        B_.dfl_set_timed_kernel(dr.handle, k)
        step()
        torch.cuda.synchronize()
        ms, n, by = B_.dfl_read_kernel_time(dr.handle)
        if n:
            breakdown[k] = {"ms": round(ms, 4), "launches": n, "GBps": round(by / (ms * 1e-3) / 1e9, 1)}
    B_.dfl_set_timed_kernel(dr.handle, -1)
    dominant = max(breakdown, key=lambda k: breakdown[k]["ms"])
    print(f"# {w.name} breakdown {json.dumps(breakdown)}", file=sys.stderr, flush=True)

    # timed region: the dominant class bracketed on the launch stream
    B_.dfl_set_timed_kernel(dr.handle, dominant)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_dom, n_dom, by_dom = B_.dfl_read_kernel_time(dr.handle)
    B_.dfl_set_timed_kernel(dr.handle, -1)
    ms_per_step = elapsed * 1e3 / steps
    value = Bq * G / (elapsed / steps)
    roofline = _roofline(dominant, d, Bq, G, ms_dom / n_dom, by_dom / n_dom, w.name, weight_kind)
    mfma = {}
    for k in ("gemm_head", "gemm_gateup"):
        # the projections as a fraction of the matrix cores' peak (the bound at large B)
        b = breakdown.get(k)
        fl = gemm_flops(k, d, Bq, G)
        if b and fl:
            mfma[k] = round(fl * b["launches"] / (b["ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)

    cpu_rec = None
    if cpu:
        print("# cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        cpu_rec = cpu_baseline(w, weights, tgt)

    out = {
        "metric": "drafted block tokens/sec (B×G) on 5-layer DFlash2; conv+walk % HBM peak",
        "value": round(value, 1),
        "unit": "block tok/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # 4-bit weights are dequantized to bf16 for the matrix units: u4 storage, bf16 arithmetic
        "dtype": "bf16" if weight_kind == "bf16" else "u4-weights/bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) taps/embeddings)",
        "config": {"workload": f"{w.name}: {d.layers}-layer drafter H={d.hidden} NH/NKV/D="
                               f"{d.heads}/{d.kv_heads}/{d.head_dim} F={d.intermediate} V={d.vocab}, "
                               f"B={Bq} G={G} L={L}" + (", 4-bit affine layer projections" if weight_kind == "q4"
                                                        else ""),
                   "B": Bq, "G": G, "L": L, "weights": weight_kind},
        "roofline": roofline,
        "mfma_frac": mfma,
        "event_breakdown_ms": {k: v["ms"] for k, v in breakdown.items()},
        "context_materialize_ms": None if ctx_ms is None else round(ctx_ms, 3),
        "cpu_baseline": cpu_rec,
    }
    if ctx_ms is not None:
        # fc + hidden norm + five k|v projections and K/V stores over B*L context rows
        T_ctx = Bq * L
        kvw = 2 * d.kv_heads * d.head_dim
        ctx_flops = 2.0 * T_ctx * d.hidden * (d.n_taps * d.hidden + d.layers * kvw)
        out["context_materialize_mfma_frac"] = round(ctx_flops / (ctx_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    dr.close()
    del weights, tgt, K, V, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def _roofline(cls, d, Bq, G, launch_ms, bytes_per_launch, workload, weight_kind):
    flops = gemm_flops(cls, d, Bq, G)
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)  # flop per byte
    if flops is not None and flops / bytes_per_launch > ridge:
        # a projection with more flops per byte than the ridge is bounded by the matrix cores
        achieved = flops / (launch_ms * 1e-3) / 1e12
        return {"kernel": cls, "bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": pmc_traffic(cls, workload, weight_kind), "avg_launch_us": round(launch_ms * 1e3, 2),
                "algorithmic_flops_per_launch": int(flops), "algorithmic_bytes_per_launch": int(bytes_per_launch)}
    achieved = bytes_per_launch / (launch_ms * 1e-3) / 1e9
    return {"kernel": cls, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": pmc_traffic(cls, workload, weight_kind), "avg_launch_us": round(launch_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": int(bytes_per_launch)}


def gemm_flops(cls: str, d, Bq: int, G: int):
    """Dense flops of one launch of a projection class (None for other classes)."""
    T, N = Bq * G, Bq * (G - 1)
    H, F, D = d.hidden, d.intermediate, d.head_dim
    ng = H // d.conv_group
    shapes = {"gemm_head": (N, d.vocab, H), "gemm_gateup": (T, 2 * F, H), "gemm_down": (T, H, F),
              "gemm_qkv": (T, (d.heads + 2 * d.kv_heads) * D, H), "gemm_o": (T, H, d.heads * D),
              "gemm_kproj": (T, 4 * ng, H), "gemm_selproj": (N, d.rank, H)}
    if cls not in shapes:
        return None
    m, n, k = shapes[cls]
    return 2.0 * m * n * k


def _time_calls(fn, steps: int, warmup: int) -> float:
    """Average milliseconds per call of fn (which enqueues on torch's current stream),
    bracketed by HIP events on that stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _time_graph(calls, replays: int, warmup: int) -> float:
    """Average milliseconds per call of a list of enqueueing closures, captured once into a
    HIP graph and replayed: events on the replay stream bracket `replays` replays, so the
    figure is GPU time per call without the host's per-call launch cost."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for fn in calls:  # eager pass before capture
            fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in calls:
            fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (replays * len(calls))


def bench_conv(steps: int, warmup: int) -> dict:
    """Grouped conv microbenchmark: T = 64 blocks of 16 rows, H = 5120, groups of 16.
    Timed: one conv application (dfl_conv_finish: the conv kernel alone, side-1 deltas
    given), the kernel projection GEMM (dfl_linear, fp32 out) and a whole dfl_conv_prepare.
    Each is captured over NSETS distinct input/output sets (more than twice the 256 MB
    Infinity Cache in total) and the graph is replayed, so every launch reads cold HBM."""
    import torch
    from dflash2_block_drafter_amd import binding as B_
    from dflash2_block_drafter_amd import configs, synth
    c = configs.CONV_BENCH
    T, H, G, grp = c["T"], c["hidden"], c["block"], c["group"]
    ng = H // grp
    nsets = 24
    sets = []
    for i in range(nsets):
        inp = synth.conv_inputs(T, H, grp, c["seed"] + i, device="cuda")
        sets.append({"x": inp["x"], "kproj": inp["kproj"], "base": inp["base"],
                     "a": torch.empty((T, H), dtype=torch.bfloat16, device="cuda"),
                     "y": torch.empty((T, H), dtype=torch.bfloat16, device="cuda"),
                     "coef1": torch.empty((T, 2 * ng), dtype=torch.float32, device="cuda"),
                     "d": torch.empty((T, 4 * ng), dtype=torch.float32, device="cuda")})
    ws = B_.workspace(max(B_.dfl_conv_prepare_workspace_bytes(T, H, grp), B_.dfl_linear_workspace_bytes(T, 4 * ng, H)))
    for st in sets:
        B_.dfl_conv_prepare(st["x"], T, H, G, grp, st["kproj"], st["base"], st["a"], st["coef1"], ws)
    torch.cuda.synchronize()
    finish = [lambda st=st: B_.dfl_conv_finish(st["a"], st["coef1"], st["base"], T, H, G, grp, None, st["y"])
              for st in sets]
    reps = max(1, steps // nsets)
    conv_ms = _time_graph(finish, reps, 2)
    # the replayed graph computes what an eager call computes
    last = sets[-1]
    eager = torch.empty_like(last["y"])
    B_.dfl_conv_finish(last["a"], last["coef1"], last["base"], T, H, G, grp, None, eager)
    torch.cuda.synchronize()
    assert torch.equal(eager, last["y"]), "graph-replayed conv differs from an eager call"
    gemm_ms = _time_graph([lambda st=st: B_.dfl_linear(st["x"], T, H, H, st["kproj"], 4 * ng, st["d"], 4 * ng, True, ws)
                           for st in sets[:8]], reps * 3, 2)
    prep_ms = _time_graph([lambda st=st: B_.dfl_conv_prepare(st["x"], T, H, G, grp, st["kproj"], st["base"], st["a"],
                                                            st["coef1"], ws) for st in sets[:8]], reps * 3, 2)
    conv_bytes = 2.0 * T * H + 4.0 * T * 2 * ng + 2.0 * 2 * H + 2.0 * T * H  # y, deltas, base side, out
    gemm_flop = 2.0 * T * 4 * ng * H
    achieved = conv_bytes / (conv_ms * 1e-3) / 1e9
    del sets, ws, eager, last
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {
        "metric": "grouped conv application time (T=1024 rows in 16-row blocks, H=5120, groups of 16)",
        "value": round(conv_ms * 1e3, 2), "unit": "us", "n_gpus": 1, "steps": reps * nsets,
        "warmup": warmup, "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "conv: T=1024 H=5120 G=16 grp=16, kernel projection 5120 -> 1280; "
                               f"{nsets} input sets rotated (cold HBM), graph-replayed launches"},
        "roofline": {"kernel": "conv_plane_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": int(conv_bytes)},
        "kernel_projection_gemm": {"us": round(gemm_ms * 1e3, 2),
                                   "tflops": round(gemm_flop / (gemm_ms * 1e-3) / 1e12, 1),
                                   "weight_GBps": round(2.0 * 4 * ng * H / (gemm_ms * 1e-3) / 1e9, 1)},
        "conv_prepare_us": round(prep_ms * 1e3, 2),
        "cpu_baseline": None,
    }


def bench_selector(steps: int, warmup: int) -> dict:
    """Candidate-selector microbenchmark: B=32 requests, S=15 slots, V=248320, K=16, R=64.
    Timed: dfl_select_tokens_projected (the selector projection in extra workgroups of the
    launch in which each row's workgroup scans its logits and takes its top-k; then edge
    scores and walk), over two input sets (0.95 GB of logits, more than the 256 MB Infinity
    Cache), captured into a HIP graph and replayed.  Also timed the same way: the
    single-step chain (compute_candidates, selector_project, score_edges, select_path in turn)."""
    import torch
    from dflash2_block_drafter_amd import binding as B_
    from dflash2_block_drafter_amd import configs, synth
    c = configs.SELECTOR_BENCH
    Bq, S, H, K, V, R = c["B"], c["S"], c["hidden"], c["top_k"], c["vocab"], c["rank"]
    N = Bq * S
    sets = []
    for i in range(2):
        inp = synth.selector_inputs(Bq, S, H, K, V, R, c["seed"] + i, device="cuda")
        sets.append({"inp": inp, "logits": inp["logits"].reshape(N, V), "hidden": inp["hidden"].reshape(N, H),
                     "ids": torch.empty((N, K), dtype=torch.int32, device="cuda"),
                     "unary": torch.empty((N, K), dtype=torch.float32, device="cuda"),
                     "z": torch.empty((N, R), dtype=torch.float32, device="cuda"),
                     "scores": torch.empty((Bq, S, K, K), dtype=torch.float32, device="cuda"),
                     "tokens": torch.empty((Bq, S), dtype=torch.int32, device="cuda")})
    ws_c = B_.workspace(B_.dfl_candidates_workspace_bytes(N, V, K))
    ws_p = B_.workspace(B_.dfl_selector_project_workspace_bytes(N, H, R))
    def fused(st):
        # the projection's workgroups run in the scan's launch (forking it onto a second
        # stream measured slower: the cross-queue fork and join cost about 20 us a chain)
        inp = st["inp"]
        B_.dfl_select_tokens_projected(st["logits"], Bq, S, V, K, st["hidden"], H, inp["proj"], R, st["z"],
                                       inp["anchors"], inp["pred"], inp["succ"], st["ids"], st["unary"],
                                       st["scores"], st["tokens"])

    def steps_chain(st):
        inp = st["inp"]
        B_.dfl_compute_candidates(st["logits"], N, V, K, st["ids"], st["unary"], ws_c)
        B_.dfl_selector_project(st["hidden"], N, H, inp["proj"], R, st["z"], ws_p)
        B_.dfl_score_edges(st["ids"], st["unary"], st["z"], inp["anchors"], Bq, S, K, R, inp["pred"], inp["succ"], V,
                           st["scores"])
        B_.dfl_select_path(st["scores"], st["ids"], Bq, S, K, st["tokens"])

    reps = max(1, steps // 2)
    ms = _time_graph([lambda st=st: fused(st) for st in sets], reps, 2)
    got = sets[-1]["tokens"].clone()
    steps_chain(sets[-1])
    torch.cuda.synchronize()
    assert torch.equal(got, sets[-1]["tokens"]), "graph-replayed selector differs from the single-step calls"
    steps_ms = _time_graph([lambda st=st: steps_chain(st) for st in sets], reps, 2)
    topk_ms = _time_graph([lambda st=st: B_.dfl_compute_candidates(st["logits"], N, V, K, st["ids"], st["unary"], ws_c)
                           for st in sets], reps, 2)
    total_bytes = 4.0 * N * V + 2.0 * N * H + 2.0 * R * H + 4.0 * N * R + 2.0 * 2 * N * K * R + 4.0 * N * K * K
    achieved = total_bytes / (ms * 1e-3) / 1e9
    del sets, ws_c, ws_p, got
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {
        "metric": "candidate selector time (B=32, S=15, V=248320, K=16, R=64): top-k + projection + edges + walk",
        "value": round(ms * 1e3, 2), "unit": "us", "n_gpus": 1, "steps": reps * 2, "warmup": warmup,
        "higher_is_better": False, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "selector: logits [32,15,248320] fp32 N(0,3), codebooks [248320,64] bf16; "
                               "2 input sets rotated, graph-replayed chain (two launches: per-row scan + "
                               "top-k with the projection beside it, then edge scores + walk)"},
        "roofline": {"kernel": "selector chain", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": int(total_bytes)},
        "single_step_chain_us": round(steps_ms * 1e3, 2),
        "compute_candidates_us": round(topk_ms * 1e3, 2),
        "cpu_baseline": None,
    }


def cpu_baseline(w, weights, tgt, budget_s: float = 10.0):
    """The CPU oracle as it stands, timed on a bounded sample of the same workload: whole
    draft blocks of requests 0, 1, ... one at a time (requests are independent), stopping
    once about `budget_s` seconds of oracle time have been spent or all requests are done.
    The sampled requests' context K/V is drawn N(0,1) at the workload's shape (the
    oracle's cost does not depend on the values)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from dflash2_block_drafter_amd import synth
    from oracle import dflash2 as O

    d = w.dims
    wh = {k: synth.host(v) for k, v in weights.items()}
    th = {k: synth.host(v) for k, v in tgt.items() if k != "taps"}
    rng = np.random.default_rng(0)
    shape = (1, w.ctx_len, d.kv_heads, d.head_dim)
    spent, done = 0.0, 0
    while done < w.batch and spent < budget_s:
        b = done
        ks = [rng.standard_normal(shape) for _ in range(d.layers)]
        vs = [rng.standard_normal(shape) for _ in range(d.layers)]
        t = time.perf_counter()
        O.draft_block(th["embeds"][b:b + 1], wh, th["lm_head"], th["anchors"][b:b + 1], ks, vs,
                      th["ctx_len"][b:b + 1], th["pos0"][b:b + 1], d)
        spent += time.perf_counter() - t
        done += 1
        print(f"# oracle block {b}: {spent:.1f} s so far", file=sys.stderr, flush=True)
    threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                  default=1)
    return {"value": round(done * d.block_size / spent, 4), "unit": "block tok/s", "cores": threads,
            "host_cpus": os.cpu_count(),
            "kind": "oracle", "seconds": round(spent, 2),
            "sample": f"whole oracle draft blocks of requests 0..{done - 1} of {w.batch} (G={d.block_size}, "
                      f"all {d.layers} layers, full V={d.vocab} head), one request per call, context K/V "
                      f"drawn N(0,1) at L={w.ctx_len}; float64 NumPy on the host"}


def calibrate_copy():
    """A plain copy of known size, for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE counters."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "torch copy_", "bytes_read": n, "bytes_written": n, "launches": 3}))


if __name__ == "__main__":
    main()
