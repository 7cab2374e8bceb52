"""Benchmark of the MoE layer forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload top2_bf16] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic tokens
already resident in HBM: route -> dispatch -> expert FFN (two grouped GEMMs)
-> combine -> aux, each through the C ABI on one stream (the flat and
hierarchical gates: the dispatch computes slots and groups, and layer 1 reads
its rows from X through row_token). W untimed warm-up
steps, then exactly K timed steps between two device synchronisations. HIP
events recorded on that same stream between the stages give every stage's
average duration; the grouped GEMM (the one dense contraction) is the
roofline kernel.

Prints one JSON line. The CPU baseline is the fp64 oracle, timed on a bounded
prefix of the same workload's tokens on the host cores.

    python bench.py --backward [--workload top2_bf16]

times a training step instead (forward, then backward: combine, expert FFN data
and weight gradients, gate and router), with the weight-gradient GEMM as the
roofline kernel.
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

PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "sparsely_gated_mixture_amd", "csrc")
TRAFFIC = {  # kernel -> (committed counter summary, the sources the kernel is built from)
    "grouped_gemm": (os.path.join(ROOT, "profiles", "grouped_gemm_top2_bf16_traffic.json"),
                     [os.path.join(CSRC, f) for f in ("gemm.hip", "common.h")]),
    "wgrad_gemm": (os.path.join(ROOT, "profiles", "wgrad_gemm_top2_bf16_traffic.json"),
                   [os.path.join(CSRC, f) for f in ("backward.hip", "common.h")]),
}


def measured_traffic(kernel: str, workload: str, layer: int | None = None):
    """HBM bytes per launch of `kernel` (of one expert layer, if given) from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated); None if absent, for
    another workload, or taken on a different version of the kernel's source."""
    import hashlib
    path, sources = TRAFFIC[kernel]
    try:
        with open(path) as f:
            t = json.load(f)
        src = b"".join(open(p, "rb").read() for p in sources)
    except OSError:
        return None
    if t.get("workload") != workload or t.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    if layer is not None:
        f, w_ = t.get(f"layer{layer}_fetch"), t.get(f"layer{layer}_write")
        return None if f is None or w_ is None else float(f) + float(w_)
    return float(t["bytes_per_launch"])


def roofline(kernel: str, flops: float, alg_bytes: float, ms: float, peak_tflops: float,
             traffic) -> dict:
    """The binding roof of a kernel: the larger of its MFMA time (flops at the dtype's
    dense peak) and its HBM time (algorithmic bytes at 8 TB/s). `achieved` and `frac`
    are against that roof; the other roof's fraction is reported beside it."""
    t_mfma = flops / (peak_tflops * 1e12)
    t_hbm = alg_bytes / (PEAK_HBM_GBS * 1e9)
    s = ms * 1e-3
    mfma = {"achieved": flops / s / 1e12, "peak": peak_tflops, "unit": "TFLOP/s"}
    hbm = {"achieved": alg_bytes / s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    bound, main, other = ("mfma", mfma, "hbm") if t_mfma >= t_hbm else ("hbm", hbm, "mfma")
    return {"bound": bound, "kernel": kernel, **main, "frac": main["achieved"] / main["peak"],
            "traffic": traffic, "traffic_unit": "bytes per launch",
            "flops_per_launch": flops, "alg_bytes_per_launch": alg_bytes, "avg_launch_ms": ms,
            f"{other}_frac": (mfma if other == "mfma" else hbm)["achieved"] /
                             (mfma if other == "mfma" else hbm)["peak"],
            "mfma_ms_at_peak": t_mfma * 1e3, "hbm_ms_at_peak": t_hbm * 1e3,
            "hbm_frac_measured": (None if traffic is None else
                                  traffic / s / 1e9 / PEAK_HBM_GBS)}


def _dev(torch, a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(a).to("cuda")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_forward_prefix(w, inp, S: int):
    from oracle import moe as O
    if w.gating == "batchwise":
        from oracle import batchwise as BO
        # the prefix as a batch of its own (m then follows the prefix size)
        BO.forward_batchwise(dict(inp, X=inp["X"][:S]), w.replace(T=S))
    elif w.groups > 0:
        from oracle import hier as HO
        # the prefix as a batch of its own (capacity, if any, then follows the prefix size)
        HO.forward_hier(dict(inp, X=inp["X"][:S]), w.replace(T=S))
    else:
        O.forward(inp, w, t_count=S)


def cpu_baseline(w, inp, budget_tokens: int, budget_tokens_1t: int):
    """The oracle as it stands on the first `budget_tokens` tokens (slots exact for a prefix)
    with every BLAS thread the host gives it, then on the first `budget_tokens_1t` tokens with
    one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    S = min(budget_tokens, w.T)
    t0 = time.perf_counter()
    _oracle_forward_prefix(w, inp, S)
    dt = time.perf_counter() - t0
    S1 = min(budget_tokens_1t, w.T)
    with threadpool_limits(1):
        t1 = time.perf_counter()
        _oracle_forward_prefix(w, inp, S1)
        dt1 = time.perf_counter() - t1
    return {"value": S / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "value_1_thread": S1 / dt1, "cpu_model": cpu_model(),
            "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"first {S} of {w.T} tokens of {w.name} on {threads} BLAS threads "
                      f"({dt:.1f} s), first {S1} on 1 thread ({dt1:.1f} s): route, slots, "
                      f"per-token expert FFN loop + combine, aux; fp64 numpy"}


def copy_probe(torch, nbytes: int, reps: int):
    """Plain device copies of a known size, for scaling HBM byte counters."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}), flush=True)


def vendor_gemm(torch, workload: str, reps: int):
    """Library batched GEMMs on the expert shapes: E groups of ceil(T*k/E) rows (capped at the
    capacity), bf16 in and out, both layers, plus one large square GEMM; median of reps."""
    from sparsely_gated_mixture_amd import inputs as I
    w = I.WORKLOADS[workload]
    dt = torch.bfloat16 if w.act == "bf16" else torch.float32
    cap = w.T if w.capacity_factor <= 0 else max(w.min_capacity, min(w.T, int(w.k * w.T * w.capacity_factor // w.E)))
    R = min(cap, -(-w.T * w.k // w.E))
    g = torch.Generator(device="cuda").manual_seed(0)
    A = torch.randn(w.E, R, w.D, device="cuda", dtype=dt, generator=g)
    W1 = torch.randn(w.E, w.D, w.H, device="cuda", dtype=dt, generator=g)
    W2 = torch.randn(w.E, w.H, w.D, device="cuda", dtype=dt, generator=g)
    Hh = torch.empty(w.E, R, w.H, device="cuda", dtype=dt)
    Z = torch.empty(w.E, R, w.D, device="cuda", dtype=dt)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        for i in range(reps):
            ev[i].record()
            fn()
        ev[reps].record()
        torch.cuda.synchronize()
        return float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))

    fl = 2.0 * w.E * R * w.D * w.H
    m1 = timed(lambda: torch.bmm(A, W1, out=Hh))
    m2 = timed(lambda: torch.bmm(Hh, W2, out=Z))
    n = 8192
    S1 = torch.randn(n, n, device="cuda", dtype=dt, generator=g)
    S2 = torch.randn(n, n, device="cuda", dtype=dt, generator=g)
    O = torch.empty_like(S1)
    m3 = timed(lambda: torch.mm(S1, S2, out=O))
    print(json.dumps({"vendor_gemm": workload, "rows_per_expert": R, "experts": w.E,
                      "layer1_ms": m1, "layer1_TFLOPs": fl / m1 / 1e9,
                      "layer2_ms": m2, "layer2_TFLOPs": fl / m2 / 1e9,
                      "square_8192_ms": m3, "square_8192_TFLOPs": 2.0 * n ** 3 / m3 / 1e9}), flush=True)


def cpu_baseline_backward(w, inp, dY, budget_tokens: int, w_imp: float, w_load: float,
                          w_switch: float = 0.0):
    """The gradient oracle as it stands on the first `budget_tokens` tokens, taken as a batch
    of their own (route, slots, fp64 autograd of the objective)."""
    from oracle import backward as OB
    from oracle import moe as O
    from oracle import philox as P
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    S = min(budget_tokens, w.T)
    ws = w.replace(T=S)
    sub = dict(inp, X=inp["X"][:S])
    t0 = time.perf_counter()
    eps = P.gaussian_noise(w.seed, S, w.E) if w.noise else None
    r = O.route(sub["X"], sub["Wg"], sub["Wnoise"], sub["bias"], w.k, w.gating, w.noise, eps=eps)
    d = O.dispatch(r.ids, w.E, O.capacity(S, w.k, w.capacity_factor, w.E, w.min_capacity))
    OB.layer_grads(sub, ws, r, d, eps, O.widen(dY[:S]), w_imp=w_imp, w_load=w_load,
                   w_switch=w_switch)
    dt = time.perf_counter() - t0
    return {"value": S / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {S} of {w.T} tokens of {w.name} as a batch of their own: route, "
                      f"slots, fp64 torch autograd of the objective (the experts those tokens "
                      f"reach); {dt:.1f} s"}


def bench_backward(args, torch, w, inp, p, L, X, t_gen):
    """A training step: the forward stages, then the backward stages, HIP events between
    them on the one stream; the weight-gradient GEMM is the roofline kernel."""
    from sparsely_gated_mixture_amd import inputs as I
    from sparsely_gated_mixture_amd import moe
    # the pages' loss weights: 0.1 for both noisy top-k terms (language models), alpha = 0.01
    # for the Switch balancing term
    sw = w.gating == "switch"
    w_imp, w_load, w_switch = (0.0, 0.0, 0.01) if sw else (0.1, 0.1, 0.0)
    dY_h = I.make_output_grad(w)
    dY = _dev(torch, dY_h)
    g = L.backward_buffers(weight_grads=True)
    b = L.b
    Hs = torch.empty_like(b.Hd) if args.recompute else None  # the recomputed activations
    hd_src = Hs if args.recompute else b.Hd
    stages = ["route", "dispatch", "gemm1", "gemm2", "combine", "aux", "combine_bwd",
              "ffn_bwd_data", "wgrad_W2", "wgrad_W1", "route_bwd"]

    def step(ev=None):
        calls = [lambda: L.route(X), lambda: L.dispatch(X), lambda: L.gemm(1),
                 lambda: L.gemm(2), lambda: L.combine(X), lambda: L.aux(),
                 lambda: L.backward_combine(dY),
                 (lambda: moe.moe_expert_ffn_backward_recompute(
                     p, b.Xd, L.W1p, g["dZ"], L.W1t, L.W2t, b.offsets, Hs, g["dHp"], g["dXd"],
                     None, None)) if args.recompute else
                 (lambda: moe.moe_expert_ffn_backward(p, b.Xd, b.Hd, g["dZ"], L.W1t, L.W2t,
                                                      b.offsets, g["dHp"], g["dXd"], None, None)),
                 lambda: moe.moe_expert_weight_grad(p, 2, hd_src, g["dZ"], b.offsets, g["dW2"]),
                 lambda: moe.moe_expert_weight_grad(p, 1, b.Xd, g["dHp"], b.offsets, g["dW1"]),
                 lambda: L.backward_route(X, dY, w_imp, w_load, w_switch=w_switch)]
        for i, c in enumerate(calls):
            if ev is not None:
                ev[i].record()
            c()
        if ev is not None:
            ev[len(calls)].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(events[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    per = {name: float(np.mean([events[s_][i].elapsed_time(events[s_][i + 1])
                                for s_ in range(args.steps)]))
           for i, name in enumerate(stages)}
    step_ev = [events[s_][0].elapsed_time(events[s_][-1]) for s_ in range(args.steps)]

    # Re-laying out the expert weights (W1, W2 into MFMA fragment order for the forward, their
    # transposes for the backward) is needed once per weight update; the training step above
    # takes the packed weights as given. Timed apart, median of 5.
    def pack_ms(fn):
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))
    repack = {"forward": pack_ms(lambda: moe.moe_pack_expert_weights(p, L.W1, L.W2, L.W1p, L.W2p)),
              "transposed": pack_ms(lambda: moe.moe_pack_expert_weights_t(p, L.W1, L.W2, L.W1t,
                                                                          L.W2t))}
    offs = b.offsets.cpu().numpy()
    A = int(offs[-1])
    U = int(np.count_nonzero(np.diff(offs)))
    el = 2 if w.act == "bf16" else 4
    flops = 2.0 * A * w.D * w.H  # per launch, either weight gradient
    wg_ms = 0.5 * (per["wgrad_W2"] + per["wgrad_W1"])
    peak = PEAK_TFLOPS[w.act]
    # per launch: both operands' rows once, the fp32 gradient of every expert written once
    wg_bytes = A * (w.D + w.H) * el + w.E * w.D * w.H * 4
    traffic = measured_traffic("wgrad_gemm", w.name)
    fwd_ms = sum(per[k] for k in stages[:6])
    bwd_ms = sum(per[k] for k in stages[6:])
    out = {
        "metric": "MoE layer fwd+bwd tokens/s at 1 GPU; weight-gradient GEMM % MFMA peak",
        "value": w.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.act,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "D": w.D, "E": w.E, "k": w.k, "H": w.H,
                   "gating": w.gating, "capacity_factor": w.capacity_factor,
                   "capacity": moe.moe_capacity(p), "accepted_rows": A, "used_experts": U,
                   "w_importance": w_imp, "w_load": w_load, "w_switch": w_switch,
                   "hidden": "recomputed in the backward" if args.recompute else "stored",
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline("wgrad_gemm", flops, wg_bytes, wg_ms, peak, traffic),
        "forward_ms": fwd_ms, "backward_ms": bwd_ms, "stages_ms": per,
        "weight_repack_ms_per_update": repack,
        "step_ms_events": {"p10": float(np.percentile(step_ev, 10)),
                           "p50": float(np.median(step_ev)),
                           "p90": float(np.percentile(step_ev, 90))},
        "input_gen_s": t_gen,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_backward(w, inp, dY_h, args.cpu_tokens_backward,
                                                    w_imp, w_load, w_switch)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="top2_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=2048)
    ap.add_argument("--cpu-tokens-1t", type=int, default=512)
    ap.add_argument("--cpu-tokens-backward", type=int, default=2048)
    ap.add_argument("--copy-probe", type=int, default=0, help="bytes; run copies only")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step of the layer instead: the forward, then the "
                         "backward (combine, expert FFN data and weight gradients, gate and "
                         "router) with w_importance = w_load = 0.1")
    ap.add_argument("--cold", action="store_true",
                    help="also time K steps each after a 512 MiB scrub write (L2 and MALL "
                         "cold), reported under 'cold'")
    ap.add_argument("--recompute", action="store_true",
                    help="with --backward: recompute the experts' hidden activations in the "
                         "backward instead of reading the forward's")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time torch.bmm (the ROCm BLAS library) on the workload's expert GEMM "
                         "shapes with a uniform rows-per-expert split, for context only")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this "
              f"single-GPU build", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    if args.copy_probe:
        copy_probe(torch, args.copy_probe, max(args.steps, 1))
        return
    if args.vendor_gemm:
        vendor_gemm(torch, args.workload, max(args.steps, 1))
        return

    from sparsely_gated_mixture_amd import inputs as I
    from sparsely_gated_mixture_amd import moe

    w = I.WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    inp = I.make_inputs(w)
    t_gen = time.perf_counter() - t_gen
    p = moe.problem(T=w.T, D=w.D, E=w.E, H=w.H, k=w.k, dtype=w.act, gating=w.gating,
                    noise=w.noise, capacity_factor=w.capacity_factor,
                    min_capacity=w.min_capacity, seed=w.seed)
    if w.gating == "batchwise":  # every expert keeps m = kT/E tokens
        L = moe.BatchwiseLayer(p, _dev(torch, inp["Wg"]), _dev(torch, inp["bias"]),
                               _dev(torch, inp["W1"]), _dev(torch, inp["W2"]))
    elif w.groups > 0:  # hierarchical gate: route / aux are the two-level stages
        L = moe.HierLayer(p, moe.hier(w.groups, w.k_primary), _dev(torch, inp["Wpg"]),
                          _dev(torch, inp["Wpn"]), _dev(torch, inp["Wsg"]),
                          _dev(torch, inp["Wsn"]), _dev(torch, inp["W1"]), _dev(torch, inp["W2"]))
    else:
        L = moe.Layer(p, _dev(torch, inp["Wg"]), _dev(torch, inp["Wnoise"]),
                      _dev(torch, inp["bias"]), _dev(torch, inp["W1"]), _dev(torch, inp["W2"]))
    X = _dev(torch, inp["X"])
    torch.cuda.synchronize()
    if args.backward:
        if w.gating not in ("noisy", "switch") or w.groups > 0:
            print("--backward covers the flat noisy top-k and Switch gates", file=sys.stderr,
                  flush=True)
            sys.exit(2)
        bench_backward(args, torch, w, inp, p, L, X, t_gen)
        return

    stages = ["route", "dispatch", "gemm1", "gemm2", "combine", "aux"]
    # flat and hierarchical gates: the dispatch computes slots and groups only and layer 1
    # reads its rows from X through row_token (the gather done by the GEMM's row loads)
    gather = isinstance(L, moe.Layer)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        L.route(X)
        if ev is not None:
            ev[1].record()
        if gather:
            L.dispatch(X, rows=False)
        else:
            L.dispatch(X)
        if ev is not None:
            ev[2].record()
        if gather:
            L.gemm(1, X)
        else:
            L.gemm(1)
        if ev is not None:
            ev[3].record()
        L.gemm(2)
        if ev is not None:
            ev[4].record()
        L.combine(X)
        if ev is not None:
            ev[5].record()
        L.aux()
        if ev is not None:
            ev[6].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    per = {name: float(np.mean([events[s][i].elapsed_time(events[s][i + 1])
                                for s in range(args.steps)]))
           for i, name in enumerate(stages)}
    step_ev = [events[s][0].elapsed_time(events[s][-1]) for s in range(args.steps)]
    cold = None
    if args.cold:
        # each step after a 512 MiB write that evicts the L2s and the MALL: weights, tokens
        # and routing state then come from HBM (event-timed steps; the scrub is not counted)
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
               for _ in range(args.steps)]
        for s in range(args.steps):
            scrub.fill_(s & 0xff)
            step(cev[s])
        torch.cuda.synchronize()
        cstep = [cev[s][0].elapsed_time(cev[s][-1]) for s in range(args.steps)]
        cold = {"scrub_bytes": 512 << 20, "step_ms_p50": float(np.median(cstep)),
                "tokens_per_s_p50": w.T / (float(np.median(cstep)) * 1e-3),
                "stages_ms": {name: float(np.mean([cev[s][i].elapsed_time(cev[s][i + 1])
                                                   for s in range(args.steps)]))
                              for i, name in enumerate(stages)}}

    def timed(fn, n):
        """Mean event time of n back-to-back launches of fn on the current stream."""
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        for i in range(n):
            ev[i].record()
            fn()
        ev[n].record()
        torch.cuda.synchronize()
        return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(n)]))

    # Outside the step: the dispatch that copies the rows into Xd (the stage of the pages'
    # dispatch the gathered layer 1 replaces), and layer 1 reading those copied rows
    copied = None
    if gather:
        n_extra = max(min(args.steps, 50), 1)
        copied = {"dispatch_ms": timed(lambda: L.dispatch(X, rows=True), n_extra),
                  "gemm1_on_Xd_ms": timed(lambda: L.gemm(1), n_extra), "launches": n_extra}

    offs = (L.st["offsets"] if w.gating == "batchwise" else L.b.offsets).cpu().numpy()
    A = int(offs[-1])
    U = int(np.count_nonzero(np.diff(offs)))  # experts that received rows
    el = 2 if w.act == "bf16" else 4
    gemm_flops = 2.0 * A * w.D * w.H  # per launch; both layers have the same count
    # per launch, either layer: the used experts' weights once, the input rows once,
    # the output rows once
    gemm_bytes = U * w.D * w.H * el + A * (w.D + w.H) * el
    peak = PEAK_TFLOPS[w.act]
    layers = {}
    for n_, name in ((1, "gemm1"), (2, "gemm2")):
        layers[name] = roofline(f"grouped_gemm layer {n_}", gemm_flops, gemm_bytes, per[name],
                                peak, measured_traffic("grouped_gemm", w.name, n_))
    slow = max(layers, key=lambda k_: per[k_])  # the headline is the slower layer
    # ids in; pos, accepted, row_token out; the rows themselves when the dispatch copies them
    slot_bytes = w.T * w.k * (4 + 4 + 1) + A * 4
    row_bytes = w.T * w.D * el + A * w.D * el
    disp_bytes = slot_bytes + (0 if gather else row_bytes)
    comb_bytes = A * w.D * el + 2 * w.T * w.D * el + w.T * w.k * 13
    out = {
        "metric": "MoE layer fwd tokens/s at 1 GPU; grouped-GEMM % MFMA peak; dispatch GB/s",
        "value": w.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.act,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "D": w.D, "E": w.E, "k": w.k, "H": w.H,
                   "gating": (f"batchwise mask, m = {w.k * w.T // w.E} tokens per expert"
                              if w.gating == "batchwise" else w.gating) if w.groups == 0 else
                   f"hierarchical {w.groups} groups x {w.E // w.groups}, k {w.k_primary} x "
                   f"{w.k // w.k_primary}",
                   "capacity_factor": w.capacity_factor,
                   "capacity": moe.moe_capacity(p), "accepted_rows": A,
                   "dropped": w.T * w.k - A, "parallelism": "none (1 GPU)"},
        "roofline": layers[slow],
        "roofline_layers": layers,
        "step_ms_events": {"p10": float(np.percentile(step_ev, 10)),
                           "p50": float(np.median(step_ev)),
                           "p90": float(np.percentile(step_ev, 90))},
        "tokens_per_s_without_aux": w.T / ((ms_per_step - per["aux"]) * 1e-3),
        "stages_ms": per,
        "dispatch_GBps": disp_bytes / (per["dispatch"] * 1e-3) / 1e9,
        "combine_GBps": comb_bytes / (per["combine"] * 1e-3) / 1e9,
        "dispatch_hbm_frac": disp_bytes / (per["dispatch"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "dispatch_rows": "gathered by layer 1's row loads" if gather else "copied into Xd",
        "combine_hbm_frac": comb_bytes / (per["combine"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "input_gen_s": t_gen,
    }
    if copied is not None:
        cb = slot_bytes + row_bytes
        out["dispatch_copying_rows"] = {
            "ms": copied["dispatch_ms"], "alg_bytes": cb,
            "GBps": cb / (copied["dispatch_ms"] * 1e-3) / 1e9,
            "hbm_frac": cb / (copied["dispatch_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "launches": copied["launches"],
            "note": "moe_dispatch with Xd: reads each token row once, writes its accepted rows"}
        out["gemm1_on_copied_rows_ms"] = copied["gemm1_on_Xd_ms"]
        out["gather_cost_in_gemm1_ms"] = per["gemm1"] - copied["gemm1_on_Xd_ms"]
    if cold is not None:
        out["cold"] = cold
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_tokens, args.cpu_tokens_1t)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
