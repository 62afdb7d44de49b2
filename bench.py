#!/usr/bin/env python3
"""Throughput of the POET layer on one MI355X: one step = build R and P, forward, backward to the skew
parameters and the AdamW update of them, for every linear of a LLaMA-shaped block, with merge-then-reinitialize
amortized over its period.

Prints one JSON line: whole-job tokens/s (inputs resident in HBM), the roofline of the dominant kernel measured
live with HIP events on the launch stream, and the CPU oracle timed on a bounded sample of the same workload.
The default run (the LLaMA-1.3B POET-BS block) also times the LLaMA-1.3B POET-FS block and reports it under
"fs_block" (skip with --no-fs), and the LLaMA-3B 24-layer POET-FS stack under "stack_3b" (skip with --no-stack).

  python bench.py [--steps K] [--warmup W] [--workload 3|4|5|2|1] [--no-cpu-baseline] [--no-fs] [--no-stack]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
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


def build_block(wl, torch, B, PI, PoetLinear, path="auto", layer=0):
    lins = []
    for lin in wl.linears(layer):
        W0, tR, tP = PI.gen_weights(wl.cfg_id, layer, lin)
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


# AdamW on the skew parameters, as a training step takes it (a small learning rate keeps the generators in the
# Neumann series' convergence range over the benchmark's few dozen steps; timing does not depend on the values)
OPTIMIZER = dict(lr=1e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


def optimizer():
    from orthogonal_reparameterized_amd import binding as B
    return B.adamw(**OPTIMIZER)


def step(lins, group=None, hp=None, pipeline=True):
    """One training step of the block: build R and P, forward, backward to the skew parameters, AdamW update.
    ``pipeline``: a group with a side class leaves that class's adjoint and update on its side stream, where they
    overlap the next step's build and the linears that do not need them (off for graph capture)."""
    hp = optimizer() if hp is None else hp
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
        group.finish_backward(join=not pipeline)
        group.optimizer_step(hp)
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
        pl.optimizer_step(hp)


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


def _prim_sums(side):
    """Sum of c^2 and of c^3 over the primitives of one side (c = block size, or s for FS)."""
    if side.mode == 1:
        return side.b ** 2, side.b ** 3
    cs = [min(side.b, side.d - o) for o in range(0, side.d, side.b)]
    return sum(c * c for c in cs), sum(c ** 3 for c in cs)


def algorithmic_flops(specs):
    """Floating-point work of one fwd+bwd step of these linears, counted on the method's definition and not on the
    kernels that run (2MNK per product):
      path A (materialize W):  6Tmn (Y, dX, weight gradient) + 2x(2n sum c_R^2 + 2m sum c_P^2) (apply + contraction)
      path B (factors on the activations):  4Tmn + 6T(sum c_R^2 + sum c_P^2)
    both plus the Cayley-Neumann chain 2k sum c^3 per side and its adjoint (twice the chain). The step's
    algorithmic MFU takes the smaller of the two, so that extra work done by the chosen path cannot raise it."""
    a = b = 0.0
    for l in specs:
        (r2, r3), (p2, p3) = _prim_sums(l.R), _prim_sums(l.P)
        chain = 2.0 * l.R.k * r3 + 2.0 * l.P.k * p3
        a += 6.0 * l.T * l.m * l.n + 2 * (2.0 * l.n * r2 + 2.0 * l.m * p2) + 3 * chain
        b += 4.0 * l.T * l.m * l.n + 6.0 * l.T * (r2 + p2) + 3 * chain
    return {"path_A": a, "path_B": b, "min": min(a, b)}


def cpu_baseline(wl, budget_s: float = 25.0, layers: int = 0):
    """The oracle (float64 NumPy, as it stands) on the same workload: forward + backward of the block's linears
    at the full token count, in order, until the time budget is spent. If it stops early, the block time is
    extrapolated from the linears done by the block's sum of m*n (and the sample string says so). A stack of
    several layers is timed on one layer and multiplied by the layer count (also said in the sample string)."""
    import numpy as np
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
        g = O.linear_bwd(sR, sP, W0, tR, tP, iR, iP, X, dY)
        for th, dth in ((tR, g["dthetaR"]), (tP, g["dthetaP"])):
            O.adamw_step(th, dth, np.zeros(len(th)), np.zeros(len(th)), 1, **OPTIMIZER)
        spent += time.perf_counter() - t0
        done.append(q)
        log(f"oracle {q.name}: {spent:.1f} s so far")
        if spent > budget_s:
            break
    scale = sum(l.m * l.n for l in lins) / sum(l.m * l.n for l in done)
    names = "+".join(l.name for l in done)
    sample = f"linears {names} forward+backward+AdamW at {wl.T} tokens in float64: {spent:.1f} s"
    if len(done) < len(lins):
        sample += f"; block time extrapolated by the block's sum of m*n ({scale:.2f}x)"
    else:
        sample += " (the whole block step)"
    layers = layers or wl.layers
    if layers > 1:
        sample += f"; one layer of {layers}, the stack's time extrapolated as {layers}x that layer"
    return {"value": round(wl.T / (spent * scale * layers), 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "sample": sample}


def _profile(B, fn, steps):
    """Run fn() `steps` times with the library's launch profiler on and return the per-class kernel records."""
    import torch
    B.poet_profile_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    prof = {B.KCLASS_NAMES[c]: B.poet_profile_query(c) for c in range(len(B.KCLASS_NAMES))}
    B.poet_profile_enable(False)
    return prof


def _timed(fn, steps, torch, join=None):
    """K calls of fn with nothing else on the stream, bracketed by synchronization; per-step event pairs on the
    current stream (the library launches on it) give the median and the minimum next to the mean. ``join`` makes
    the current stream wait for work the last step left on other streams, before the closing event."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(steps):
        fn()
        if join is not None and i == steps - 1:
            join()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]) / steps, per, wall


def _roofline(prof, peak, traffic=None):
    """Roofline line of the dominant token-GEMM class: its algorithmic flops over its launch durations."""
    token = {k: prof[k] for k in ("token_fwd", "token_dx", "token_gw")}
    dom = max(token, key=lambda k: token[k]["ms"])
    d = token[dom]
    achieved = d["flops"] / (d["ms"] / 1e3) / 1e12 if d["ms"] > 0 else 0.0
    return dom, {"bound": "mfma", "kernel": f"gemm ({dom})", "achieved": round(achieved, 1), "peak": peak,
                 "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                 "avg_launch_ms": round(d["ms"] / max(d["launches"], 1), 4), "launches": d["launches"],
                 "flops_per_launch": d["flops"] / max(d["launches"], 1)}


def mfma_probe(torch, B, workgroups: int = 2048, iters: int = 1024, warm_launches: int = 100):
    """The bf16 matrix-core rate this GPU sustains (poet_mfma_probe: MFMAs on registers only, eight waves per
    workgroup, eight rounds of workgroups per CU), timed with events on the current stream, the library's launch
    stream: the ceiling that the clock held under full matrix load leaves a GEMM, next to the published peak. The
    clock rises only under sustained load (a burst of 1 ms after idle runs about a fifth slower), so about 100 ms of
    probe launches run first; the median of the next 9 is reported."""
    out = torch.empty(workgroups * 8, dtype=torch.float32, device="cuda")
    for _ in range(warm_launches):
        B.poet_mfma_probe(iters, workgroups, out)
    torch.cuda.synchronize()
    times, flops = [], 0.0
    for _ in range(9):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = B.poet_mfma_probe(iters, workgroups, out)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    tf = flops / (ms / 1e3) / 1e12
    return {"achieved": round(tf, 1), "unit": "TFLOP/s", "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "ms_median": round(ms, 4), "workgroups": workgroups, "mfma_per_wave": 4 * iters}


def _hbm_class(p):
    """Achieved GB/s of a data-movement kernel class on its algorithmic bytes."""
    if not p["launches"] or p["ms"] <= 0:
        return None
    gbs = p["bytes"] / (p["ms"] / 1e3) / 1e9
    return {"ms": round(p["ms"], 4), "launches": p["launches"], "algorithmic_bytes": p["bytes"],
            "achieved_GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}


def _merge_leg(B, torch, build, merge, nbytes, period):
    """Merge-then-reinitialize of every linear, timed on its own and amortized over its period. Each of three
    merges follows a build (untimed: the merge folds built factors); the first pays each kernel's first load, the
    second is timed, the third runs under the launch profiler."""
    ms_merge, mprof = None, None
    for rep in range(3):
        build()
        torch.cuda.synchronize()
        B.poet_profile_enable(rep == 2)
        m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m0.record()
        merge()
        m1.record()
        torch.cuda.synchronize()
        if rep == 1:
            ms_merge = m0.elapsed_time(m1)
    mprof = {B.KCLASS_NAMES[c]: B.poet_profile_query(c) for c in range(len(B.KCLASS_NAMES))}
    B.poet_profile_enable(False)
    info = {"ms_all_linears": round(ms_merge, 4), "algorithmic_bytes": nbytes,
            "achieved_GBps": round(nbytes / (ms_merge / 1e3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms_merge / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "kernel_ms": {k: round(v["ms"], 4) for k, v in mprof.items() if v["launches"]},
            "kernel_launches": {k: v["launches"] for k, v in mprof.items() if v["launches"]}}
    mk = _hbm_class(mprof["merge"])
    if mk is not None:
        info["merge_kernels"] = mk
    return ms_merge, info


def side_linears(lins, args):
    """The MLP linears of a POET-BS block (their sides are the same size as the attention linears', so no class of
    sizes sets them apart): the group's side stream takes them, last in the step order."""
    if args.side_linears == "none" or args.no_side_chains:
        return None
    from orthogonal_reparameterized_amd import binding as B
    if not all(e["pl"].L.R.mode == B.POET_BS and e["pl"].L.P.mode == B.POET_BS for e in lins):
        return None
    names = ("gate", "up", "down") if args.side_linears == "mlp" else tuple(args.side_linears.split(","))
    idx = [i for i, e in enumerate(lins) if e["spec"].name in names]
    return idx if 0 < len(idx) < len(lins) else None


def block_group(lins, PoetGroup, args):
    """The group the benchmark steps a block with (None with --no-group); linears whose FS pair the group forms
    keep their W there."""
    if args.no_group:
        return None
    group = PoetGroup([e["pl"] for e in lins], form_fs=not args.no_form, form_streams=args.form_streams,
                      side_chains=not args.no_side_chains, side_linears=side_linears(lins, args))
    for e in lins:
        if id(e["pl"]) in group._formed:
            e["keep"] = None
    return group


def run_block(wl, args, torch, B, PI, PoetLinear, PoetGroup):
    """One block of 7 linears (or the single-linear workload): timed steps, profiled steps, merge leg."""
    log(f"workload {wl.name}: allocating")
    lins = build_block(wl, torch, B, PI, PoetLinear, args.path)
    group = block_group(lins, PoetGroup, args)
    pipe = not args.no_pipeline
    torch.cuda.synchronize()
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step(lins, group, pipeline=pipe)
    torch.cuda.synchronize()

    # one step captured into a HIP graph (torch's CUDAGraph over the HIP stream the library launches on): replays
    # issue the same kernels with the same arguments without the host's per-launch cost
    graph = None
    if args.graph:
        log("capturing one step into a graph")
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            step(lins, group, pipeline=False)  # a step on the capture stream first (the library's first launch on
            # a stream)
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(lins, group, pipeline=False)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()

    log(f"timed {args.steps} steps")
    run = (lambda: graph.replay()) if graph is not None else (lambda: step(lins, group, pipeline=pipe))
    ms_step, per, wall = _timed(run, args.steps, torch, join=group.join if group is not None else None)
    # the same K steps again with the library's launch profiler on (an event pair around every launch, on the
    # launch stream): per-class kernel times and the dominant kernel's launch duration. The events add gaps
    # between launches, not kernel time, so this pass is kept out of the timed region above.
    log(f"profiled {args.steps} steps")
    prof = _profile(B, lambda: step(lins, group, pipeline=pipe), args.steps)

    log("merge")
    # algorithmic HBM bytes: every element of W0 read and written once in float32, plus the bf16 copy of W0 the
    # activation-side path reads, written by the same merge
    merge_bytes = sum((10.0 if e["pl"].act_path else 8.0) * e["spec"].m * e["spec"].n for e in lins)
    if group is not None:
        ms_merge, merge_info = _merge_leg(B, torch, group.build, group.merge, merge_bytes, args.merge_period)
    else:
        def build_all():
            for e in lins:
                e["pl"].build()

        def merge_all():
            for e in lins:
                e["pl"].merge()
        ms_merge, merge_info = _merge_leg(B, torch, build_all, merge_all, merge_bytes, args.merge_period)

    ms_total = ms_step + ms_merge / args.merge_period
    peak = PEAK_BF16_TFLOPS if wl.dtype == PI.DT_BF16 else PEAK_F32_TFLOPS
    act = all(e["pl"].act_path for e in lins)
    dom, roof = _roofline(prof, peak)
    if wl.cfg_id == 3 and act:
        roof["traffic"] = measured_traffic(dom)
    token = [prof[k] for k in ("token_fwd", "token_dx", "token_gw")]
    gemm_ms, gemm_fl = sum(v["ms"] for v in token), sum(v["flops"] for v in token)
    fl = algorithmic_flops([e["spec"] for e in lins])
    res = {
        "value": round(wl.T / (ms_total / 1e3), 1), "ms_per_step": round(ms_total, 4),
        "ms_fwd_bwd": round(ms_step, 4), "ms_fwd_bwd_median": round(statistics.median(per), 4),
        "ms_fwd_bwd_min": round(min(per), 4), "ms_merge_all_linears": round(ms_merge, 4),
        "config": {"workload": wl.name, "hidden": wl.hidden, "ffn": wl.ffn, "tokens": wl.T,
                   "mode": "BS" if wl.mode == PI.MODE_BS else "FS",
                   "block": wl.b, "fraction": wl.frac, "k": wl.k, "linears": len(lins),
                   "factor_application": "activations" if act else
                   ("weight" if not any(e["pl"].act_path for e in lins) else "mixed"),
                   "grouped_side_steps": group is not None, "merge_period": args.merge_period,
                   "fs_formed_in_build": bool(group is not None and group._formed),
                   "form_streams": len(group._form_streams) if group is not None else 0,
                   "side_chain_sides": len(group._side_idx) if group is not None else 0,
                   "side_class_pipelined": bool(group is not None and group._side_idx and pipe and not args.graph)},
        "roofline": roof, "merge": merge_info, "host_wall_s": round(wall, 3), "graph_replay": graph is not None,
        "kernel_ms_per_step": round(sum(v["ms"] for v in prof.values()) / args.steps, 4),
        "token_gemm_tflops": round(gemm_fl / (gemm_ms / 1e3) / 1e12, 1) if gemm_ms else None,
        "algorithmic_tflop_per_step": {k: round(v / 1e12, 4) for k, v in fl.items()},
        "step_mfu": round(fl["min"] / (ms_total / 1e3) / 1e12 / peak, 4),
        "stage_ms_per_step": {k: round(v["ms"] / args.steps, 4) for k, v in prof.items()},
        "stage_launches_per_step": {k: v["launches"] // args.steps for k, v in prof.items()},
    }
    g = _hbm_class({k: v / args.steps if k != "launches" else v // args.steps for k, v in prof["gather"].items()})
    if g is not None:
        res["gather_scatter"] = g
    del lins, group, graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def run_stack(wl, args, torch, B, PI, PoetLinear, PoetGroup):
    """A stack of `layers` LLaMA blocks with every layer's state resident at once: float32 W0 (and the bf16 copy the
    activation side reads), skew parameters with their gradients and AdamW moments, primitives and operand copies,
    saved Neumann powers, index sets, and what each linear keeps for its backward (the layer inputs, and Z on the
    activation side or the materialized W on the weight side). One step = grouped build and forward of every layer
    in order, then in reverse order the backward of every layer to the primitive gradients, the grouped adjoint and
    the AdamW update. Weights and activations are drawn on the device with the recipe's distributions (W0
    row-normalized Gaussian, theta ~ N(0, 1e-3^2), X and dY ~ N(0, 1) in bf16). Inputs of one shape are shared the
    way a transformer layer shares them (q/k/v read one input, gate/up one).

    Store or recompute (--recompute): "powers" keeps one set of saved-power buffers for all layers and rebuilds each
    layer's factors before its backward (a second Cayley-Neumann chain per layer instead of k saved powers per side);
    "weights" lets the weight-side backward form W = R W0 P again instead of keeping it from the forward."""
    T = wl.T
    nl = args.layers or wl.layers
    rec = set(x for x in args.recompute.split(",") if x and x != "none")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    specs = [wl.linears(layer) for layer in range(nl)]
    shapes = specs[0]
    ws_lin = max(PoetLinear.workspace_bytes(l.m, l.n, T, B.side_of(l.R), B.side_of(l.P), l.act_dtype,
                                            PI.pad_ld(l.n), PI.pad_ld(l.n), PI.pad_ld(l.m), args.path) for l in shapes)
    ws = torch.empty(ws_lin, dtype=torch.uint8, device="cuda")
    wide = max(PI.pad_ld(max(l.m, l.n)) for l in shapes)
    Ybuf = torch.empty((T, wide), dtype=torch.bfloat16, device="cuda")
    dXbuf = torch.empty((T, wide), dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 * wl.cfg_id + 17)
    dYs = {}  # one upstream gradient per output width, shared by the layers
    for l in shapes:
        ldy = PI.pad_ld(l.m)
        if ldy not in dYs:
            dYs[ldy] = torch.randn((T, ldy), generator=g, device="cuda").to(torch.bfloat16)
    share = {"q": "attn", "k": "attn", "v": "attn", "o": "o", "gate": "mlp", "up": "mlp", "down": "down"}
    mem = dict.fromkeys(("W0_f32", "W0_bf16_copy", "theta_grad_moments", "primitives_and_operand_copies",
                         "saved_powers", "index_sets", "kept_inputs", "kept_Z_or_W", "folded_weights",
                         "fs_gradient_operands", "workspaces_and_transients"), 0)
    # FS pairs formed in the group build (W and the gradient operands kept from the build to the backward), unless
    # W is formed again in the backward
    form = not args.no_form and "weights" not in rec
    shared_pw = {}  # position in the layer -> saved-power buffers reused by every layer (recompute "powers")
    layers = []
    for layer, lins in enumerate(specs):
        xs, es = {}, []
        for j, lin in enumerate(lins):
            W0 = torch.randn((lin.m, lin.n), generator=g, device="cuda")
            W0 /= W0.norm(dim=1, keepdim=True)
            tR = torch.randn(B.poet_theta_len(B.side_of(lin.R)), generator=g, device="cuda") * PI.THETA_STD
            tP = torch.randn(B.poet_theta_len(B.side_of(lin.P)), generator=g, device="cuda") * PI.THETA_STD
            ldx, ldy = PI.pad_ld(lin.n), PI.pad_ld(lin.m)
            pl = PoetLinear(lin.m, lin.n, T, B.side_of(lin.R), B.side_of(lin.P), lin.act_dtype, W0, tR, tP,
                            seed=wl.seed, linear_id=lin.linear_id, ldw=PI.pad_ld(lin.n), ldx=ldx, ldy=ldy, ws=ws,
                            path=args.path)
            del W0, tR, tP
            if "powers" in rec:
                if j not in shared_pw:
                    shared_pw[j] = (pl.powersR, pl.powersP)
                else:
                    pl.powersR, pl.powersP = shared_pw[j]
            key = share[lin.name]
            if key not in xs:
                xs[key] = torch.randn((T, ldx), generator=g, device="cuda").to(torch.bfloat16)
                mem["kept_inputs"] += _nbytes(xs[key])
            keep = None
            if pl.act_path:
                keep = pl.alloc_act(T, ldy)  # Z = X P^T W0^T
            elif "weights" not in rec and not (form and PoetGroup._formable(pl)):
                keep = pl.alloc_W()
            mem["kept_Z_or_W"] += _nbytes(keep)
            mem["W0_f32"] += _nbytes(pl.W0)
            mem["W0_bf16_copy"] += _nbytes(pl.W0b)
            mem["theta_grad_moments"] += sum(_nbytes(t) for t in (pl.thetaR, pl.thetaP, pl.dthetaR, pl.dthetaP, pl.mR,
                                                                  pl.mP, pl.vR, pl.vP))
            mem["primitives_and_operand_copies"] += sum(_nbytes(t) for t in (pl.primR, pl.primP, pl.qnormR,
                                                                             pl.qnormP))
            if "powers" not in rec or layer == 0:
                mem["saved_powers"] += _nbytes(pl.powersR) + _nbytes(pl.powersP)
            mem["index_sets"] += _nbytes(pl.idxR) + _nbytes(pl.idxP)
            es.append({"spec": lin, "pl": pl, "X": xs[key], "keep": keep,
                       "Y": Ybuf.view(-1)[:T * ldy].view(T, ldy), "dX": dXbuf.view(-1)[:T * ldx].view(T, ldx),
                       "dY": dYs[ldy]})
        layers.append(es)
        log(f"stack: layer {layer} allocated, {torch.cuda.memory_allocated() / 2**30:.1f} GiB")
    sl = side_linears(layers[0], args)
    gws = torch.empty(max(PoetGroup.workspace_bytes([e["pl"] for e in layers[0]], not args.no_side_chains, sl), 1),
                      dtype=torch.uint8, device="cuda")
    fws = None  # the formation streams' workspaces, shared by the groups (their builds run one after another)
    if form:
        fneed = PoetGroup.form_workspace_bytes([e["pl"] for e in layers[0]])
        if fneed:
            fws = [torch.empty(fneed, dtype=torch.uint8, device="cuda") for _ in range(args.form_streams)]
    side = None  # the side stream and its workspace, shared by the groups (their calls run one after another)
    sneed = PoetGroup.side_workspace_bytes([e["pl"] for e in layers[0]], sl)
    if sneed and not args.no_side_chains:
        side = (torch.cuda.Stream(), torch.empty(sneed, dtype=torch.uint8, device="cuda"))
    groups = [PoetGroup([e["pl"] for e in es], ws=gws, form_fs=form, form_streams=args.form_streams, form_ws=fws,
                        side_chains=not args.no_side_chains, side=side, side_linears=sl)
              for es in layers]
    for grp in groups:  # the group's operand copies, folded weights and formed FS operands
        for W, Zr, Acp in grp._formed.values():
            mem["kept_Z_or_W"] += _nbytes(W)
            mem["fs_gradient_operands"] += _nbytes(Zr) + _nbytes(Acp)
        for v in grp._ops.values():
            mem["primitives_and_operand_copies"] += sum(_nbytes(t) for t in v)
        for v in grp._fold.values():
            mem["folded_weights"] += sum(_nbytes(t) for t in v)
    state_bytes = torch.cuda.memory_allocated() - base
    mem["workspaces_and_transients"] = state_bytes - sum(mem.values())
    hp = optimizer()

    def fwd(e):
        pl = e["pl"]
        if pl.act_path:
            pl.forward_act(e["X"], e["Y"], e["keep"])
        else:
            pl.forward(e["X"], e["Y"], W_out=e["keep"])

    def bwd(e):
        pl = e["pl"]
        if pl.act_path:
            pl.backward_act_prims(e["X"], e["keep"], e["dY"], e["dX"])
        else:
            pl.backward_prims(e["X"], e["dY"], e["dX"], W=e["keep"])

    def stack_step():
        for es, grp in zip(layers, groups):
            grp.build()
            for e in es:
                fwd(e)
        for es, grp in zip(reversed(layers), reversed(groups)):
            if "powers" in rec:  # the saved powers were overwritten by later layers: form them again
                grp.build(again=True)
            for e in reversed(es):
                bwd(e)
            grp.finish_backward(join=args.no_pipeline)
            grp.optimizer_step(hp)

    log(f"stack warmup {args.warmup}")
    for _ in range(args.warmup):
        stack_step()
    torch.cuda.synchronize()
    log(f"stack timed {args.steps} steps")
    ms_step, per, wall = _timed(stack_step, args.steps, torch, join=lambda: [grp.join() for grp in groups])
    log("stack profiled step")
    prof = _profile(B, stack_step, 1)
    log("stack merge")
    all_specs = [e["spec"] for es in layers for e in es]
    merge_bytes = sum((10.0 if e["pl"].act_path else 8.0) * e["spec"].m * e["spec"].n for es in layers for e in es)

    def build_all():
        for grp in groups:
            grp.build()

    def merge_all():
        for grp in groups:
            grp.merge()
    ms_merge, merge_info = _merge_leg(B, torch, build_all, merge_all, merge_bytes, args.merge_period)
    ms_total = ms_step + ms_merge / args.merge_period
    peak_bytes = torch.cuda.max_memory_allocated() - base
    n_params = sum(l.m * l.n for l in all_specs)
    n_theta = sum(B.poet_theta_len(B.side_of(l.R)) + B.poet_theta_len(B.side_of(l.P)) for l in all_specs)
    fl = algorithmic_flops(all_specs)
    dom, roof = _roofline(prof, PEAK_BF16_TFLOPS)
    act = all(e["pl"].act_path for es in layers for e in es)
    gib = 1.0 / 2 ** 30
    res = {
        "value": round(T / (ms_total / 1e3), 1), "ms_per_step": round(ms_total, 4), "ms_fwd_bwd": round(ms_step, 4),
        "ms_fwd_bwd_median": round(statistics.median(per), 4), "ms_fwd_bwd_min": round(min(per), 4),
        "ms_merge_all_linears": round(ms_merge, 4),
        "config": {"workload": wl.name if nl == wl.layers else f"{wl.name}_x{nl}layers", "hidden": wl.hidden,
                   "ffn": wl.ffn, "tokens": T, "mode": "BS" if wl.mode == PI.MODE_BS else "FS", "block": wl.b,
                   "fraction": wl.frac, "k": wl.k, "layers": nl, "linears": len(all_specs),
                   "factor_application": "activations" if act else "weight", "grouped_side_steps": True,
                   "merge_period": args.merge_period, "recompute": sorted(rec) or ["none"],
                   "fs_formed_in_build": form and any(grp._formed for grp in groups),
                   "side_chain_sides": sum(len(grp._side_idx) for grp in groups),
                   "side_class_pipelined": not args.no_pipeline and any(grp._side_idx for grp in groups)},
        "roofline": roof, "merge": merge_info, "host_wall_s": round(wall, 3),
        "algorithmic_tflop_per_step": {k: round(v / 1e12, 4) for k, v in fl.items()},
        "step_mfu": round(fl["min"] / (ms_total / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "stage_ms_per_step": {k: round(v["ms"], 4) for k, v in prof.items()},
        # device memory: the measured peak of the whole run and the resident state before the first step, by kind
        # (every allocation of the run, summed from the tensors' sizes); for comparison, the weight-state of dense
        # AdamW training of the same linears: float32 weight, its gradient and the two moments, 16 bytes per weight
        # element (arithmetic, not measured; the activations a layer keeps are the same for both)
        "memory": {"peak_hbm_gib": round(peak_bytes * gib, 2), "resident_state_gib": round(state_bytes * gib, 2),
                   "resident_by_kind_gib": {k: round(v * gib, 3) for k, v in mem.items()},
                   "linear_weight_elements": n_params, "trainable_skew_params": n_theta,
                   "poet_weight_state_gib": round((mem["W0_f32"] + mem["W0_bf16_copy"] + mem["theta_grad_moments"])
                                                  * gib, 2),
                   "dense_adamw_weight_grad_moments_gib": round(16.0 * n_params * gib, 2)},
    }
    g = _hbm_class(prof["gather"])
    if g is not None:
        res["gather_scatter"] = g
    del layers, groups
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def parser():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--layers", type=int, default=0,
                    help="run the workload's block as a stack of this many layers, all resident (the LLaMA-3B "
                         "workload is a 24-layer stack by default)")
    ap.add_argument("--recompute", default="none",
                    help="with a stack: comma-separated parts formed again in the backward instead of kept from "
                         "the forward: powers (the saved Neumann powers), weights (the materialized W)")
    ap.add_argument("--merge-period", type=int, default=400)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fs", action="store_true",
                    help="with the default workload, skip the extra LLaMA-1.3B POET-FS block measurement")
    ap.add_argument("--no-stack", action="store_true",
                    help="with the default workload, skip the extra LLaMA-3B 24-layer POET-FS stack measurement")
    ap.add_argument("--stack-steps", type=int, default=5,
                    help="timed steps of the extra LLaMA-3B stack measurement (its warmup is 2 steps)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured into a HIP graph (the default launches every step)")
    ap.add_argument("--path", default="auto", choices=["auto", "weight", "act"],
                    help="apply R and P to the activations around the W0 GEMM (act), materialize W (weight), or "
                         "the activation side wherever it is supported (auto)")
    ap.add_argument("--no-group", action="store_true",
                    help="build and finish the backward of each linear on its own (the default runs the per-side "
                         "steps of all linears of the block in shared launches)")
    ap.add_argument("--no-form", action="store_true",
                    help="form W and the FS gradient operands in each linear's forward and backward (the default "
                         "forms them for every weight-side POET-FS linear in the group build, overlapped on side "
                         "streams)")
    ap.add_argument("--form-streams", type=int, default=1,
                    help="side streams the group build forms the FS pairs on")
    ap.add_argument("--no-pipeline", action="store_true",
                    help="join the side class's adjoint at the end of the backward (the default leaves it and the "
                         "class's AdamW update running on the side stream into the next step)")
    ap.add_argument("--side-linears", default="mlp",
                    help="POET-BS blocks: the linears that build, fold and run their adjoint on the side stream: "
                         "mlp (gate, up, down), none, or a comma-separated list of names (POET-FS blocks take their "
                         "wide primitives there by size)")
    ap.add_argument("--no-side-chains", action="store_true",
                    help="build and differentiate all sides of a group in one call per step (the default runs the "
                         "class of large primitives with the most product work, e.g. the MLP's s = 2730 POET-FS "
                         "sides, on a side stream beside the rest)")
    ap.add_argument("--permuted", action="store_true",
                    help="permuted POET-BS: each side's blocks on a random permutation, fresh at every merge "
                         "(PermutedPoetLinear; implies --no-group and skips the extra FS block)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB 3 times (a plain copy kernel of known size "
                         "that calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    return ap


def main():
    args = parser().parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the POET layer path is single-GPU (data-parallel sharding is a "
              "design note only); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import poet_inputs as PI
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.layer import PermutedPoetLinear, PoetGroup, PoetLinear
    if args.permuted:
        if PI.WORKLOADS[args.workload].mode != PI.MODE_BS or args.layers > 1 or PI.WORKLOADS[args.workload].layers > 1:
            print("--permuted applies to the one-block POET-BS workloads (1, 2, 3)", file=sys.stderr)
            sys.exit(2)
        args.no_group, args.no_fs = True, True
        PoetLinear = PermutedPoetLinear

    torch.cuda.set_device(0)
    B.lib()
    wl = PI.WORKLOADS[args.workload]
    if (args.layers or wl.layers) > 1:
        res = run_stack(wl, args, torch, B, PI, PoetLinear, PoetGroup)
    else:
        res = run_block(wl, args, torch, B, PI, PoetLinear, PoetGroup)
    out = {"metric": METRIC, "value": res.pop("value"), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": res.pop("ms_per_step"), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.dtype == PI.DT_BF16 else "f32",
           "data": "synthetic", "config": res.pop("config"), "roofline": res.pop("roofline")}
    out.update(res)
    out["config"]["permuted_blocks"] = bool(args.permuted)
    if args.workload == 3 and args.layers <= 1 and not args.no_fs:
        fs = PI.WORKLOADS[4]
        log("extra: the POET-FS block")
        r4 = run_block(fs, args, torch, B, PI, PoetLinear, PoetGroup)
        out["fs_block"] = {"unit": "tokens/s", **r4}
    if args.workload == 3 and args.layers <= 1 and not args.no_stack and not args.permuted:
        # the LLaMA-3B 24-layer POET-FS stack at 32768 tokens, every layer resident (about 72 GiB), with fewer
        # steps than the block: one step takes about half a second
        log("extra: the LLaMA-3B 24-layer POET-FS stack")
        sargs = argparse.Namespace(**vars(args))
        sargs.steps, sargs.warmup, sargs.layers = max(1, args.stack_steps), min(args.warmup, 2), 0
        r5 = run_stack(PI.WORKLOADS[5], sargs, torch, B, PI, PoetLinear, PoetGroup)
        out["stack_3b"] = {"unit": "tokens/s", "steps": sargs.steps, "warmup": sargs.warmup, **r5}
    log("matrix-core probe")
    out["mfma_probe"] = mfma_probe(torch, B)
    for r in [out["roofline"]] + [out[k]["roofline"] for k in ("fs_block", "stack_3b") if k in out]:
        if r.get("peak") == PEAK_BF16_TFLOPS and out["mfma_probe"]["achieved"] > 0:
            r["frac_of_sustained"] = round(r["achieved"] / out["mfma_probe"]["achieved"], 4)
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
        out["cpu_baseline"] = cpu_baseline(wl, layers=args.layers)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
