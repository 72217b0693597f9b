#!/usr/bin/env python3
"""Benchmark of the exact top-k indexer selection path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM: hytopk_select (sampled threshold, fused score +
compare + compaction, check, recovery / full rescore when needed, candidate
select + sort) followed by hytopk_replay of the selected indices.

Default workload: the GLM-5.1-shaped one-GPU shard of the HyScale explainer's
worked example (L = 1,048,576 keys, n = 8,192 queries at the last positions,
H = 64, d = 128, k = 2,048, bf16 q/k ~ N(0,1)/sqrt(d), fp32 w ~ U(0,1)/H).

Prints ONE JSON line.  value = algorithmic TFLOP/s of the step (2*H*d per
causal pair for selection plus 2*H*d per replayed entry) / step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "mxfp8": 5033.2, "mxfp4": 10066.3}  # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "HyTopK select ms + TFLOP/s (%MFMA peak) at L=1M,n=8192,k=2048; replay ms"
def traffic_file(workload: str) -> str:
    """Stored HBM counters of the score kernel for a workload (profiles/)."""
    name = "glm1m_bf16" if workload == "glm1m" else workload
    return os.path.join(ROOT, "profiles", f"traffic_score_tile_{name}.txt")
KERNEL_SOURCES = ["exact_top_token_amd/csrc/score.hip", "exact_top_token_amd/csrc/tile.h",
                  "exact_top_token_amd/csrc/common.h"]


def kernel_hash() -> str:
    """Hash of the score kernel's sources with comments and blank space
    removed: stored HBM counters stay valid across comment-only edits and
    become stale on any change to the code."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def scoring_flops(L: int, n: int, H: int, d: int, q_start: int) -> float:
    pairs = sum_ctx(q_start, n)
    return 2.0 * H * d * pairs


def sum_ctx(q_start: int, n: int) -> int:
    return n * (q_start + 1) + n * (n - 1) // 2


def replay_bytes(n, H, d, k, fmt) -> int:
    """Algorithmic bytes of replay: per entry the key row (+ its scales), the
    index and the output score; per query its rows (+ scales) and weights."""
    row = {"bf16": 2 * d, "fp8": d, "mxfp8": d + d // 32, "mxfp4": d // 2 + d // 32}[fmt]
    tok = 4 if fmt == "fp8" else 0   # per-token fp32 scale
    per_entry = row + tok + 4 + 4
    per_query = H * (row + 4) + tok
    return n * k * per_entry + n * per_query


def backward_bytes(L, n, H, d, k, fmt="bf16") -> int:
    """Algorithmic HBM bytes of the backward: per entry the key row in its
    storage format (+ its per-token scale), its index and upstream gradient;
    per query its rows and weights read, dq and dw written; dk written once."""
    row = {"bf16": 2 * d, "fp8": d, "mxfp8": d + d // 32, "mxfp4": d // 2 + d // 32}[fmt]
    tok = 4 if fmt == "fp8" else 0
    per_entry = row + tok + 4 + 4
    per_query = H * (row + 4) + tok + H * (d * 4 + 4)
    return n * k * per_entry + n * per_query + L * d * 4


def cpu_baseline(inp, seconds_target: float = 15.0) -> dict:
    """The oracle as it stands, on a bounded sample of the same workload: the
    fp64 decode of the keys is built once (outside the timed loop), then each
    sampled query is scored over its whole context and its exact top-k taken
    (``oracle.score_row`` + ``oracle.exact_topk``), which is the oracle's
    per-query selection work."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    dec = oracle.Decoded(inp)
    t_decode = time.perf_counter() - t0
    sub = []
    flops = 0.0
    i = inp.n - 1
    step = max(1, inp.n // 97)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds_target and i >= 0 and len(sub) < 256:
        oracle.exact_topk(oracle.score_row(dec, i), inp.k)
        ctx = inp.L - inp.n + i + 1
        flops += 2.0 * inp.H * inp.d * ctx
        sub.append(i)
        i -= step
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"oracle.score_row + oracle.exact_topk (fp64 numpy/BLAS scores over the "
                      f"whole context, exact lexsort top-k) on {len(sub)} queries of the same "
                      f"workload (every {step}th from the last), {dt:.1f} s; the fp64 key decode "
                      f"({t_decode:.1f} s, once per problem) is not timed; full call "
                      f"extrapolated: {dt / len(sub) * inp.n:.0f} s"}


def device_inputs(inp, dev: str) -> dict:
    """The workload's storage arrays as device tensors (argument marshalling
    only: the bytes are the ones datagen wrote)."""
    import numpy as np
    import torch
    fmt = inp.dtype
    if fmt == "fp8":
        q = torch.from_numpy(inp.q).to(dev).view(torch.float8_e4m3fn)
        k = torch.from_numpy(inp.k_).to(dev).view(torch.float8_e4m3fn)
        qs = torch.from_numpy(inp.q_scale).to(dev)
        ks = torch.from_numpy(inp.k_scale).to(dev)
    elif fmt in ("mxfp8", "mxfp4"):
        q = torch.from_numpy(inp.q).to(dev)
        k = torch.from_numpy(inp.k_).to(dev)
        qs = torch.from_numpy(inp.q_scale).to(dev)
        ks = torch.from_numpy(inp.k_scale).to(dev)
    else:
        q = torch.from_numpy(inp.q.view(np.int16)).to(dev).view(torch.bfloat16)
        k = torch.from_numpy(inp.k_.view(np.int16)).to(dev).view(torch.bfloat16)
        qs = ks = None
    w = torch.from_numpy(inp.w).to(dev)
    fk = dict(fmt=fmt) if fmt in ("mxfp8", "mxfp4") else {}
    return dict(q=q, k=k, w=w, qs=qs, ks=ks, fk=fk)


def time_select_replay(hk, inp, t: dict, steps: int, warmup: int) -> dict:
    """Warm up, then time `steps` steps of select + replay on the current
    stream: whole-region events, per-call events, and the library's own event
    pairs around each of its launches (per-phase averages)."""
    import numpy as np
    import torch
    dev = t["q"].device
    q, k, w, qs, ks, fk = t["q"], t["k"], t["w"], t["qs"], t["ks"], t["fk"]
    ws = torch.empty(hk.select_workspace_bytes(q, k, w, inp.k, **fk), dtype=torch.uint8, device=dev)
    idx = torch.empty((inp.n, inp.k), dtype=torch.int32, device=dev)
    sc = torch.empty((inp.n, inp.k), dtype=torch.float32, device=dev)
    rep = torch.empty_like(sc)
    for _ in range(warmup):
        hk.select(q, k, w, inp.k, q_scale=qs, k_scale=ks, workspace=ws, out=(idx, sc), **fk)
        hk.replay(q, k, w, idx, q_scale=qs, k_scale=ks, out=rep, **fk)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    hk.trace_enable(True)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    stats = None
    for i in range(steps):
        ev[i][0].record()
        _, _, stats = hk.select(q, k, w, inp.k, q_scale=qs, k_scale=ks, workspace=ws,
                                out=(idx, sc), with_stats=True, **fk)
        ev[i][1].record()
        hk.replay(q, k, w, idx, q_scale=qs, k_scale=ks, out=rep, **fk)
        ev[i][2].record()
    t_end.record()
    torch.cuda.synchronize()
    phases = hk.trace_read()
    hk.trace_enable(False)
    del ws
    return dict(ms_per_step=t_start.elapsed_time(t_end) / steps,
                select_ms=float(np.median([a.elapsed_time(b) for a, b, _ in ev])),
                replay_ms=float(np.median([b.elapsed_time(c) for _, b, c in ev])),
                phases=phases, stats=stats, idx=idx, sc=sc)


def time_graph_step(hk, inp, t: dict, steps: int, ref_idx, ref_sc) -> dict:
    """The same step (select + replay) recorded once in a HIP graph through
    hytopk_select_async (no host synchronisation), then replayed `steps`
    times.  The replays' outputs must equal the eager calls' bit for bit."""
    import torch
    dev = t["q"].device
    q, k, w, qs, ks, fk = t["q"], t["k"], t["w"], t["qs"], t["ks"], t["fk"]
    ws = torch.empty(hk.select_workspace_bytes(q, k, w, inp.k, **fk), dtype=torch.uint8, device=dev)
    idx = torch.empty((inp.n, inp.k), dtype=torch.int32, device=dev)
    sc = torch.empty((inp.n, inp.k), dtype=torch.float32, device=dev)
    rep = torch.empty_like(sc)
    status = torch.zeros(hk.ASYNC_STATUS_WORDS, dtype=torch.int32, device=dev)

    def step():
        hk.select_async(q, k, w, inp.k, q_scale=qs, k_scale=ks, workspace=ws, out=(idx, sc),
                        status=status, **fk)
        hk.replay(q, k, w, idx, q_scale=qs, k_scale=ks, out=rep, **fk)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # outside the capture: the library sets its kernels' LDS limits once
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    equal = bool(torch.equal(idx, ref_idx) and torch.equal(sc.view(torch.int32), ref_sc.view(torch.int32)))
    st = status.cpu().tolist()
    del g, ws, idx, sc, rep, status
    torch.cuda.empty_cache()
    return {"ms_per_step": round(a.elapsed_time(b) / steps, 4), "equal_to_eager": equal,
            "failures": st[1], "incomplete": st[0]}


def workload_summary(inp, m: dict) -> dict:
    """Per-workload figures: select and replay times, and the fused score
    kernel against the MFMA peak of the workload's format."""
    q_start = inp.L - inp.n
    sel_flops = scoring_flops(inp.L, inp.n, inp.H, inp.d, q_start)
    peak = PEAK_TFLOPS[inp.dtype]
    c, tot = m["phases"].get("score_compact", (0, 0.0))
    score_ms = tot / max(1, c)
    rbytes = replay_bytes(inp.n, inp.H, inp.d, inp.k, inp.dtype)
    return {"workload": f"L={inp.L} n={inp.n} H={inp.H} d={inp.d} k={inp.k} {inp.dtype}",
            "select_ms": round(m["select_ms"], 4),
            "select_tflops": round(sel_flops / (m["select_ms"] * 1e-3) / 1e12, 2),
            "score_ms": round(score_ms, 4),
            "score_tflops": round(sel_flops / (score_ms * 1e-3) / 1e12, 2) if score_ms else None,
            "score_peak_frac": round(sel_flops / (score_ms * 1e-3) / 1e12 / peak, 4) if score_ms else None,
            "peak_tflops": peak,
            "replay_ms": round(m["replay_ms"], 4),
            "replay_gbs": round(rbytes / (m["replay_ms"] * 1e-3) / 1e9, 1),
            "replay_hbm_frac": round(rbytes / (m["replay_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "phases_ms": {nm: round(t / max(1, n), 4) for nm, (n, t) in m["phases"].items()},
            "n_failed": (m["stats"] or {}).get("n_failed")}


EXTRA_WORKLOADS = ("glm1m_fp8", "mid")  # measured in the same run, reported beside the headline


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="glm1m", help="datagen config name")
    ap.add_argument("--no-baseline", action="store_true", help="skip the score-table baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the indexer backward at the replayed entries")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-recorded step (hytopk_select_async + replay)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra workloads (" + ", ".join(EXTRA_WORKLOADS) + ")")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run one plain device-to-device copy of BYTES bytes (calibrates "
                         "the HBM byte counters of a profiler run) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the selection path has no multi-GPU mode (each "
              "GPU would select for its own query shard after an all-gather of the keys); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_probe:
        torch.cuda.set_device(0)
        x = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda:0")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe}), flush=True)
        return 0

    import datagen
    import exact_top_token_amd as hk

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    torch.cuda.set_device(0)
    dev = "cuda:0"
    hk.load_library()
    log(f"generating {args.workload}")
    inp = datagen.make(args.workload)
    fmt = inp.dtype
    t = device_inputs(inp, dev)
    q, k, w, qs, ks, fk = t["q"], t["k"], t["w"], t["qs"], t["ks"], t["fk"]

    log(f"warmup {args.warmup}, timing {args.steps} steps")
    m = time_select_replay(hk, inp, t, args.steps, args.warmup)
    idx, sc = m["idx"], m["sc"]
    summ = workload_summary(inp, m)
    ms_per_step = m["ms_per_step"]
    select_ms, replay_ms = m["select_ms"], m["replay_ms"]

    q_start = inp.L - inp.n
    sel_flops = scoring_flops(inp.L, inp.n, inp.H, inp.d, q_start)
    rep_flops = 2.0 * inp.H * inp.d * inp.n * inp.k
    peak = PEAK_TFLOPS[fmt]
    value = (sel_flops + rep_flops) / (ms_per_step * 1e-3) / 1e12

    score_ms = summ["score_ms"]
    achieved = sel_flops / (score_ms * 1e-3) / 1e12 if score_ms > 0 else None

    traffic = None
    if os.path.exists(traffic_file(args.workload)):
        try:
            tr = json.load(open(traffic_file(args.workload)))
            if tr.get("kernel_hash") == kernel_hash() and tr.get("workload") == args.workload:
                traffic = tr.get("bytes_per_launch")
        except Exception:
            traffic = None

    baseline_ms = None
    if not args.no_baseline:
        log("baseline: materialise the score table, then row top-k")
        bws = torch.empty(hk.baseline_workspace_bytes(q, k, w, inp.k, **fk), dtype=torch.uint8, device=dev)
        bidx = torch.empty_like(idx)
        bsc = torch.empty_like(sc)
        hk.baseline_select(q, k, w, inp.k, q_scale=qs, k_scale=ks, workspace=bws, out=(bidx, bsc),
                           **fk)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        hk.baseline_select(q, k, w, inp.k, q_scale=qs, k_scale=ks, workspace=bws, out=(bidx, bsc),
                           **fk)
        b.record()
        torch.cuda.synchronize()
        baseline_ms = a.elapsed_time(b)
        same = bool(torch.equal(bidx, idx) and torch.equal(bsc.view(torch.int32), sc.view(torch.int32)))
        del bws, bidx, bsc
        if not same:
            log("WARNING: baseline result differs from hytopk_select")

    graph = None
    if not args.no_graph:
        log(f"graph: select_async + replay recorded once, {args.steps} replays")
        graph = time_graph_step(hk, inp, t, args.steps, idx, sc)
        if not graph["equal_to_eager"]:
            log("WARNING: graph-replayed result differs from hytopk_select")

    bwd = None
    if not args.no_backward:
        log("backward at the replayed entries (dq, dw, dk)")
        bk = dict(fmt=fmt, q_scale=qs, k_scale=ks) if fmt != "bf16" else {}
        bws = torch.empty(hk.backward_workspace_bytes(q, k, w, inp.k, **fk), dtype=torch.uint8,
                          device=dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(1234)
        dsc = torch.randn((inp.n, inp.k), generator=gen, dtype=torch.float32, device=dev)
        outs = {"dq": torch.empty((inp.n, inp.H, inp.d), dtype=torch.float32, device=dev),
                "dw": torch.empty((inp.n, inp.H), dtype=torch.float32, device=dev),
                "dk": torch.empty((inp.L, inp.d), dtype=torch.float32, device=dev)}
        for _ in range(max(1, args.warmup)):
            hk.backward(q, k, w, idx, dsc, workspace=bws, out=outs, **bk)
        torch.cuda.synchronize()
        hk.trace_enable(True)
        bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in bev:
            a.record()
            hk.backward(q, k, w, idx, dsc, workspace=bws, out=outs, **bk)
            b.record()
        torch.cuda.synchronize()
        bph = hk.trace_read()
        hk.trace_enable(False)
        bms = float(np.median([a.elapsed_time(b) for a, b in bev]))
        abytes = backward_bytes(inp.L, inp.n, inp.H, inp.d, inp.k, fmt)
        bwd = {"ms": round(bms, 4), "algorithmic_bytes": abytes,
               "gbs": round(abytes / (bms * 1e-3) / 1e9, 1),
               "hbm_frac": round(abytes / (bms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
               "phases_ms": {nm: round(tt / args.steps, 4) for nm, (c, tt) in bph.items()}}
        del bws, outs, dsc

    cpu = None
    if not args.no_cpu:
        log("cpu baseline: oracle on a bounded sample")
        cpu = cpu_baseline(inp, args.cpu_seconds)

    stats = m["stats"]
    del t, q, k, w, qs, ks, idx, sc, m
    torch.cuda.empty_cache()
    extra = {}
    if not args.no_extra:
        for name in EXTRA_WORKLOADS:
            if name == args.workload:
                continue
            log(f"extra workload {name}: generating, then {max(3, min(args.steps, 10))} steps")
            xi = datagen.make(name)
            xt = device_inputs(xi, dev)
            xm = time_select_replay(hk, xi, xt, max(3, min(args.steps, 10)), max(1, min(args.warmup, 2)))
            extra[name] = workload_summary(xi, xm)
            del xt, xm
            torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8_e4m3", "mxfp8": "mxfp8_e4m3", "mxfp4": "mxfp4_e2m1"}[fmt],
        "data": "synthetic (seeded datagen; no dataset or weights)",
        "config": {"workload": f"{args.workload}: L={inp.L} n={inp.n} (positions {q_start}..{inp.L - 1}) "
                               f"H={inp.H} d={inp.d} k={inp.k}",
                   "L": inp.L, "n": inp.n, "H": inp.H, "d": inp.d, "k": inp.k,
                   "parallelism": "single GPU"},
        "select_ms": round(select_ms, 4),
        "select_tflops": summ["select_tflops"],
        "select_mfma_frac": round(summ["select_tflops"] / peak, 4),
        "replay_ms": round(replay_ms, 4),
        "replay_gbs": summ["replay_gbs"],
        "replay_hbm_frac": summ["replay_hbm_frac"],
        "baseline_ms": None if baseline_ms is None else round(baseline_ms, 3),
        "baseline_over_select": None if baseline_ms is None else round(baseline_ms / select_ms, 3),
        "phases_ms": summ["phases_ms"],
        "backward": bwd,
        "graph": graph,
        "stats": stats,
        "extra_workloads": extra or None,
        "roofline": {"bound": "mfma", "kernel": "score_tile_kernel (fused score+compare+compact)",
                     "achieved": None if achieved is None else round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": None if achieved is None else round(achieved / peak, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
