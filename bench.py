#!/usr/bin/env python3
"""Throughput of the POET layer on one MI355X: one step = build R and P, forward, and backward to the skew
parameters for every linear of a LLaMA-shaped block, with merge-then-reinitialize amortized over its period.

Prints one JSON line: whole-job tokens/s (inputs resident in HBM), the roofline of the dominant kernel measured
live with HIP events on the launch stream, and the CPU oracle timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload 3|4|2|1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "POET layer fwd+bwd tokens/s at LLaMA-1.3B shapes (bf16); % MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU (the published 2.5 PFLOP/s)
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def build_block(wl, torch, B, PI, PoetLinear, path="auto"):
    lins = []
    for lin in wl.linears(0):
        W0, tR, tP = PI.gen_weights(wl.cfg_id, 0, lin)
        ldw, ldx, ldy = PI.pad_ld(lin.n), PI.pad_ld(lin.n), PI.pad_ld(lin.m)
        pl = PoetLinear(lin.m, lin.n, lin.T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP,
                        seed=wl.seed, linear_id=lin.linear_id, ldw=ldw, ldx=ldx, ldy=ldy, path=path)
        g = torch.Generator(device="cuda")
        g.manual_seed(1000 * wl.cfg_id + lin.linear_id)
        X = torch.randn((lin.T, ldx), generator=g, device="cuda", dtype=torch.float32).to(pl.act)
        dY = torch.randn((lin.T, ldy), generator=g, device="cuda", dtype=torch.float32).to(pl.act)
        # the tensor the forward keeps for the backward: Z = X P^T W0^T (activation-side path) or W
        keep = pl.alloc_act(lin.T, ldy) if pl.act_path else pl.alloc_W()
        lins.append({"spec": lin, "pl": pl, "X": X, "dY": dY, "Y": pl.alloc_act(lin.T, ldy),
                     "dX": pl.alloc_act(lin.T, ldx), "keep": keep})
    return lins


def step(lins, group=None):
    if group is not None:  # the block's per-side steps in shared launches: build, then per linear, then adjoint
        group.build()
        for e in lins:
            pl = e["pl"]
            if pl.act_path:
                pl.forward_act(e["X"], e["Y"], e["keep"])
                pl.backward_act_prims(e["X"], e["keep"], e["dY"], e["dX"])
            else:
                pl.forward(e["X"], e["Y"], W_out=e["keep"])
                pl.backward_prims(e["X"], e["dY"], e["dX"], W=e["keep"])
        group.finish_backward()
        return
    for e in lins:
        pl = e["pl"]
        pl.build()
        if pl.act_path:
            pl.forward_act(e["X"], e["Y"], e["keep"])
            pl.backward_act(e["X"], e["keep"], e["dY"], e["dX"])
        else:
            pl.forward(e["X"], e["Y"], W_out=e["keep"])
            pl.backward(e["X"], e["dY"], e["dX"], W=e["keep"])


def measured_traffic(tag: str):
    """HBM bytes per launch of a token-GEMM class from the committed rocprofv3 counter summary of this workload,
    or None when the summary is missing, is for another kernel class, or was taken on a different version of the
    GEMM source (its sha256 no longer matches)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "token_gemm_traffic_llama1.3b_bs256.json")
    try:
        doc = json.load(open(path))
        src = open(os.path.join(ROOT, doc["source"]), "rb").read()
        if hashlib.sha256(src).hexdigest() != doc["source_sha256"]:
            return None
        return doc["kernels"][tag]["traffic_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def algorithmic_flops(lins):
    """2MNK of the three token GEMMs of every linear (Y, dX and the weight gradient)."""
    return sum(3 * 2.0 * e["spec"].T * e["spec"].m * e["spec"].n for e in lins)


def cpu_baseline(wl, budget_s: float = 25.0):
    """The oracle (float64 NumPy, as it stands) on the same workload: forward + backward of the block's linears
    at the full token count, in order, until the time budget is spent. If it stops early, the block time is
    extrapolated from the linears done by the block's sum of m*n (and the sample string says so)."""
    import oracle as O
    import poet_inputs as PI
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    lins = wl.linears(0)
    spent, done = 0.0, []
    for q in lins:
        W0, tR, tP, X, dY = PI.gen_linear(wl.cfg_id, 0, q)
        iR = O.sample_indices(q.m, q.R.b, wl.seed, q.linear_id, O.SIDE_R, 0) if q.R.mode == PI.MODE_FS else None
        iP = O.sample_indices(q.n, q.P.b, wl.seed, q.linear_id, O.SIDE_P, 0) if q.P.mode == PI.MODE_FS else None
        sR, sP = O.Side.of(q.R), O.Side.of(q.P)
        t0 = time.perf_counter()
        O.linear_fwd(sR, sP, W0, tR, tP, iR, iP, X)
        O.linear_bwd(sR, sP, W0, tR, tP, iR, iP, X, dY)
        spent += time.perf_counter() - t0
        done.append(q)
        log(f"oracle {q.name}: {spent:.1f} s so far")
        if spent > budget_s:
            break
    scale = sum(l.m * l.n for l in lins) / sum(l.m * l.n for l in done)
    names = "+".join(l.name for l in done)
    sample = f"linears {names} forward+backward at {wl.T} tokens in float64: {spent:.1f} s"
    if len(done) < len(lins):
        sample += f"; block time extrapolated by the block's sum of m*n ({scale:.2f}x)"
    else:
        sample += " (the whole block step)"
    return {"value": round(wl.T / (spent * scale), 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": sample}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4])
    ap.add_argument("--merge-period", type=int, default=400)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured into a HIP graph (the default launches every step)")
    ap.add_argument("--path", default="auto", choices=["auto", "weight", "act"],
                    help="apply R and P to the activations around the W0 GEMM (act), materialize W (weight), or "
                         "the activation side wherever it is supported (auto)")
    ap.add_argument("--no-group", action="store_true",
                    help="build and finish the backward of each linear on its own (the default runs the per-side "
                         "steps of all linears of the block in shared launches)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB 3 times (a plain copy kernel of known size "
                         "that calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the POET layer path is single-GPU (data-parallel sharding is a "
              "design note only); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import poet_inputs as PI
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PoetGroup, PoetLinear

    torch.cuda.set_device(0)
    B.lib()
    wl = PI.WORKLOADS[args.workload]
    log(f"workload {wl.name}: allocating")
    lins = build_block(wl, torch, B, PI, PoetLinear, args.path)
    group = None if args.no_group else PoetGroup([e["pl"] for e in lins])
    torch.cuda.synchronize()
    T = wl.T

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step(lins, group)
    torch.cuda.synchronize()

    # one step captured into a HIP graph (torch's CUDAGraph over the HIP stream the library launches on): replays
    # issue the same kernels with the same arguments without the host's per-launch cost
    graph = None
    if args.graph:
        log("capturing one step into a graph")
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            step(lins, group)  # a step on the capture stream first (the library's first launch on a stream)
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(lins, group)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()

    # timed region: K steps (graph replays, or eager launches) with nothing else on the stream
    log(f"timed {args.steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step(lins, group)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    # the same K steps again with the library's launch profiler on (an event pair around every launch, on the
    # launch stream): per-class kernel times and the dominant kernel's launch duration. The events add gaps
    # between launches, not kernel time, so this pass is kept out of the timed region above.
    log(f"profiled {args.steps} steps")
    B.poet_profile_enable(True)
    for _ in range(args.steps):
        step(lins, group)
    torch.cuda.synchronize()
    prof = {B.KCLASS_NAMES[c]: B.poet_profile_query(c) for c in range(len(B.KCLASS_NAMES))}
    B.poet_profile_enable(False)

    # merge-then-reinitialize of every linear, timed on its own and amortized over its period; its kernels are
    # profiled separately (algorithmic HBM bytes: every element of W0 read and written once, float32)
    # (one untimed merge first: the first call of each kernel pays its load; the work of a merge does not depend
    # on the state it leaves, and a third, profiled merge gives the per-class kernel times)
    log("merge")
    for rep in range(3):
        torch.cuda.synchronize()
        B.poet_profile_enable(rep == 2)
        m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m0.record()
        if group is not None:
            group.merge()
        else:
            for e in lins:
                e["pl"].merge()
        m1.record()
        torch.cuda.synchronize()
        if rep == 1:
            ms_merge = m0.elapsed_time(m1)
    mprof = {B.KCLASS_NAMES[c]: B.poet_profile_query(c) for c in range(len(B.KCLASS_NAMES))}
    B.poet_profile_enable(False)
    # (plus the bf16 copy of W0 the activation-side path reads, written by the same merge)
    merge_bytes = sum((10.0 if e["pl"].act_path else 8.0) * e["spec"].m * e["spec"].n for e in lins)
    merge_info = {"ms_all_linears": round(ms_merge, 4), "algorithmic_bytes": merge_bytes,
                  "achieved_GBps": round(merge_bytes / (ms_merge / 1e3) / 1e9, 1),
                  "hbm_frac": round(merge_bytes / (ms_merge / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                  "kernel_ms": {k: round(v["ms"], 4) for k, v in mprof.items() if v["launches"]},
                  "kernel_launches": {k: v["launches"] for k, v in mprof.items() if v["launches"]}}

    ms_total = ms_step + ms_merge / args.merge_period
    tokens_per_s = T / (ms_total / 1e3)

    # roofline of the dominant kernel class
    token = {k: prof[k] for k in ("token_fwd", "token_dx", "token_gw")}
    dom = max(token, key=lambda k: token[k]["ms"])
    d = token[dom]
    avg_ms = d["ms"] / max(d["launches"], 1)
    achieved = d["flops"] / (d["ms"] / 1e3) / 1e12 if d["ms"] > 0 else 0.0
    peak = PEAK_BF16_TFLOPS if wl.dtype == PI.DT_BF16 else PEAK_F32_TFLOPS
    gemm_ms = sum(v["ms"] for v in token.values())
    gemm_fl = sum(v["flops"] for v in token.values())

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_total, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == PI.DT_BF16 else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "hidden": wl.hidden, "ffn": wl.ffn, "tokens": T,
                   "mode": "BS" if wl.mode == PI.MODE_BS else "FS",
                   "block": wl.b, "fraction": wl.frac, "k": wl.k, "linears": len(lins),
                   "factor_application": "activations" if all(e["pl"].act_path for e in lins) else
                   ("weight" if not any(e["pl"].act_path for e in lins) else "mixed"),
                   "grouped_side_steps": group is not None, "merge_period": args.merge_period},
        "roofline": {"bound": "mfma", "kernel": f"gemm ({dom})", "achieved": round(achieved, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(dom) if wl.cfg_id == 3 and all(e["pl"].act_path for e in lins) else None,
                     "avg_launch_ms": round(avg_ms, 4), "launches": d["launches"],
                     "flops_per_launch": d["flops"] / max(d["launches"], 1)},
        "ms_fwd_bwd": round(ms_step, 4), "ms_merge_all_linears": round(ms_merge, 4), "merge": merge_info,
        "host_wall_s": round(wall, 3), "graph_replay": graph is not None,
        "kernel_ms_per_step": round(sum(v["ms"] for v in prof.values()) / args.steps, 4),
        "token_gemm_tflops": round(gemm_fl / (gemm_ms / 1e3) / 1e12, 1) if gemm_ms else None,
        "step_mfu": round(algorithmic_flops(lins) / (ms_total / 1e3) / 1e12 / peak, 4),
        "stage_ms_per_step": {k: round(v["ms"] / args.steps, 4) for k, v in prof.items()},
        "stage_launches_per_step": {k: v["launches"] // args.steps for k, v in prof.items()},
    }
    if args.calib_copy_mib > 0:
        nbytes = args.calib_copy_mib << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = nbytes
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
