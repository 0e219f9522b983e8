#!/usr/bin/env python3
"""Benchmark of the EQ-Linear spectral forward on one MI355X.

A step is one eqlin_forward over one batch of the workload (the whole hot path: load, group DFT,
per-frequency products, inverse DFT + bias, store -- one fused kernel). Default workload: p4
(G = 4), C_in = C_out = 96, N = 8x56x56 = 25088 tokens, bf16 in/out, synthetic seeded inputs.

Timing. Inputs are resident in HBM before the timed region. W warmup steps run eagerly; then K steps
are captured into one HIP graph (so the ~10 us kernels are not bounded by host launch latency) and
replayed once untimed and once timed, between HIP events on the launch stream, with
torch.cuda.synchronize() on both sides. The K steps rotate over R buffer sets totalling >= 1 GiB,
more than the 256 MB Infinity Cache, so x is read from HBM, not from the cache.
ms_per_step = event time / K; value = tokens / (ms_per_step / 1e3).

Per-launch median and minimum come from a separate pass of eager launches, each between its own
pair of events. The same is done for eqlin_forward_expanded (the unrolled dense product, the
comparator); torch's F.linear on the unrolled weight is timed as context only; and the fp64 oracle
is timed on the host cores over a bounded sample (cpu_baseline, with a one-thread figure).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "EQ-Linear fwd tokens/s + % of bf16 MFMA/HBM roofline vs expanded dense GEMM"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def load_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from fourier_domain_linear_amd.profiling import kernel_source_hash

    if rec.get("source_sha256") != kernel_source_hash():
        log(f"[bench] {path} was taken on other kernel sources: traffic = null")
        return None
    return rec.get("traffic_bytes_per_launch")


def time_graph(torch, launch, K: int, R: int):
    """Capture K launches (launch(i) uses buffer set i % R) into one graph; replay once untimed and
    once timed. Returns ms per launch."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            launch(i % R)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / K


def time_eager(torch, launch, K: int, R: int):
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        launch(i % R)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / K


def time_each(torch, launch, n: int, R: int):
    """Per-launch durations: n eager launches, each between its own pair of events on the launch
    stream (the pair adds a little to each figure). Returns {"median", "min"} in microseconds."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, e) in enumerate(ev):
        a.record(stream)
        launch(i % R)
        e.record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(e) * 1e3 for a, e in ev)
    return {"median": round(us[n // 2], 3), "min": round(us[0], 3), "launches": n,
            "timing": "eager launches, an event pair around each"}


def cpu_baseline(w, x, W, b, budget_s: float = 12.0):
    """The fp64 oracle, as it stands, on the host cores over a bounded sample of the workload: whole
    passes over the workload's tokens until about `budget_s` seconds have run, or (when one pass
    would take longer) the first tokens that fit the budget, sized by a pilot run."""
    import oracle

    threads = oracle.max_threads()
    fwd = oracle.dihedral.forward if w.group == "d4" else oracle.forward  # D4: numpy's matmul (its BLAS threads)
    pilot = min(w.N, 256)
    t0 = time.perf_counter()
    fwd(x[:pilot], W, b)
    per_token = (time.perf_counter() - t0) / pilot
    if per_token * w.N <= budget_s / 2:
        passes, t0 = 0, time.perf_counter()
        while passes < 1000 and time.perf_counter() - t0 < budget_s:
            fwd(x, W, b)
            passes += 1
        dt = time.perf_counter() - t0
        tokens = passes * w.N
        sample = f"{passes} pass(es) over all {w.N} tokens of the workload"
    else:
        n = min(w.N, max(pilot, int(budget_s / per_token)))
        t0 = time.perf_counter()
        fwd(x[:n], W, b)
        dt = time.perf_counter() - t0
        tokens = n
        sample = f"first {n} of {w.N} tokens of the workload"
    out = {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle", "sample": sample,
           "seconds": round(dt, 3), "cpu_model": _cpu_model()}
    if w.group != "d4":
        # the same oracle on one thread, over the first tokens that fit about a quarter of the budget
        t0 = time.perf_counter()
        fwd(x[:pilot], W, b, threads=1)
        n1 = min(w.N, max(pilot, int(budget_s / 4 / max(1e-12, (time.perf_counter() - t0) / pilot))))
        t0 = time.perf_counter()
        fwd(x[:n1], W, b, threads=1)
        out["single_thread"] = {"value": n1 / (time.perf_counter() - t0), "unit": "tokens/s",
                                "sample": f"first {n1} of {w.N} tokens"}
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_block(torch, eq, rl, timer, dev, K: int, Wm: int, with_expanded: bool):
    """Time the MLP block (layer 1 with GELU in its epilogue, then layer 2; two launches per step) on
    its seeded inputs, its two layers alone, and the same block on the unrolled weights."""
    from fourier_domain_linear_amd.workloads import BLOCK_WORKLOAD as bw, make_block_inputs

    G, C, H, N, eb = bw.G, bw.C_in, bw.C_out, bw.N, bw.elem_bytes
    log(f"[bench] block {bw.name}: G={G} C={C} hidden={H} N={N} {bw.dtype}")
    x, W1, b1, W2, b2 = make_block_inputs(G, C, H, N, bw.dtype, seed=0)
    set_bytes = N * (C + H + C) * G * eb
    R = max(3, math.ceil((1 << 30) / set_bytes))
    x0 = x.to(dev)
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    hs = [torch.empty((N, H, G), dtype=bw.torch_dtype, device=dev) for _ in range(R)]
    ys = [torch.empty((N, C, G), dtype=bw.torch_dtype, device=dev) for _ in range(R)]
    h1 = eq.prepare_weights(W1.to(dev), expanded=with_expanded)
    h2 = eq.prepare_weights(W2.to(dev), expanded=with_expanded)
    b1d, b2d = b1.to(dev), b2.to(dev)
    torch.cuda.synchronize()
    steps = {
        "block": lambda i: eq.mlp_block(h1, b1d, h2, b2d, xs[i], hs[i], ys[i]),
        "layer1_gelu": lambda i: eq.forward(h1, xs[i], b1d, hs[i], act="gelu"),
        "layer1_plain": lambda i: eq.forward(h1, xs[i], b1d, hs[i]),
        "layer2": lambda i: eq.forward(h2, hs[i], b2d, ys[i]),
    }
    if with_expanded:
        steps["expanded_block"] = lambda i: eq.mlp_block(h1, b1d, h2, b2d, xs[i], hs[i], ys[i], expanded=True)
    ms = {}
    for name, fn in steps.items():
        for i in range(Wm):
            fn(i % R)
        torch.cuda.synchronize()
        ms[name] = timer(torch, fn, K, R)
        log(f"[bench] block {name}: {ms[name] * 1e3:.2f} us/step")
    F = rl.spectral_flops(N, C, H, G) + rl.spectral_flops(N, H, C, G)
    Fd = rl.dense_flops(N, C, H, G) + rl.dense_flops(N, H, C, G)
    t = ms["block"] / 1e3
    res = {"workload": bw.name, "ms_per_step": round(ms["block"], 6), "tokens_per_s": N / t,
           "useful_tflops": round(F / t / 1e12, 2), "effective_tflops": round(Fd / t / 1e12, 2),
           "mfma_frac": round(F / t / 1e12 / rl.PEAK_BF16_TFLOPS, 4),
           "layers_ms": {k: round(v, 6) for k, v in ms.items() if k != "block" and k != "expanded_block"},
           "gelu_epilogue_us": round((ms["layer1_gelu"] - ms["layer1_plain"]) * 1e3, 2),
           "kernels": [h1.describe(), h2.describe()]}
    if with_expanded:
        te = ms["expanded_block"] / 1e3
        res["expanded_block"] = {"ms_per_step": round(ms["expanded_block"], 6), "tokens_per_s": N / te,
                                 "effective_tflops": round(Fd / te / 1e12, 2)}
        res["speedup_vs_expanded"] = round(ms["expanded_block"] / ms["block"], 3)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None, help="workload name (default: the p4, 96-channel one)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-expanded", action="store_true")
    ap.add_argument("--json-out", default=None, help="also write the JSON line to this file")
    ap.add_argument("--backward", action="store_true",
                    help="also time eqlin_backward_data and eqlin_backward_weights (reported under 'backward')")
    ap.add_argument("--block", action="store_true",
                    help="also time the transformer MLP block EQ-Linear(C->4C), GELU, EQ-Linear(4C->C) at the "
                         "p4 192-channel shape, spectral and expanded (reported under 'block')")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (the counter calibration for traffic)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch

        a = torch.ones(args.calibrate_copy, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(max(1, args.steps)):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": args.calibrate_copy, "launches": max(1, args.steps)}))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the layer is token-parallel "
              "with no communication: N GPUs would each run this on N-th of the tokens).", file=sys.stderr)
        sys.exit(2)

    import torch

    import fourier_domain_linear_amd as eq
    from fourier_domain_linear_amd import roofline as rl
    from fourier_domain_linear_amd.workloads import BENCH_WORKLOAD, BY_NAME, make_grad, workload_inputs

    w = BY_NAME[args.workload] if args.workload else BENCH_WORKLOAD
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    eq.load_library()

    log(f"[bench] workload {w.name}: G={w.G} C_in={w.C_in} C_out={w.C_out} N={w.N} {w.dtype}")
    x, W, b = workload_inputs(w, seed=0)
    eb = w.elem_bytes
    set_bytes = w.N * (w.C_in + w.C_out) * w.G * eb
    R = max(3, math.ceil((1 << 30) / set_bytes))
    xd0 = x.to(dev)
    xs = [xd0] + [xd0.clone() for _ in range(R - 1)]
    ys = [torch.empty((w.N, w.C_out, w.G), dtype=w.torch_dtype, device=dev) for _ in range(R)]
    bd = b.to(dev)
    h = eq.prepare_weights(W.to(dev), expanded=not args.no_expanded, backward=args.backward, group=w.group)
    torch.cuda.synchronize()
    log(f"[bench] {h.describe()}  rotating buffer sets: {R} ({R * set_bytes / 2**20:.0f} MiB)")

    def spectral(i):
        eq.forward(h, xs[i], bd, ys[i])

    def expanded(i):
        eq.forward_expanded(h, xs[i], bd, ys[i])

    K, Wm = args.steps, args.warmup
    timer = time_eager if args.no_graph else time_graph
    for i in range(Wm):
        spectral(i % R)
    torch.cuda.synchronize()
    ms = timer(torch, spectral, K, R)
    log(f"[bench] spectral: {ms * 1e3:.2f} us/step")

    F = rl.spectral_flops(w.N, w.C_in, w.C_out, w.G, w.group)
    B = rl.spectral_bytes(w.N, w.C_in, w.C_out, w.G, eb)
    # fp16 matrix cores have the bf16 dense peak on this chip (2.5 PFLOP/s)
    peak_c = rl.PEAK_BF16_TFLOPS if w.dtype in ("bf16", "f16") else rl.PEAK_FP32_TFLOPS
    _, bound = rl.roof_time_s(F, B, peak_c)
    t = ms / 1e3
    if bound == "hbm":
        achieved, peak, unit = B / t / 1e9, rl.PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = F / t / 1e12, peak_c, "TFLOP/s"
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": load_traffic(w.name),
            "kernel": "spectral forward (one launch per step)",
            "algorithmic_bytes_per_launch": B, "algorithmic_flops_per_launch": F,
            "mfma_frac": round(F / t / 1e12 / peak_c, 4), "hbm_frac": round(B / t / 1e9 / rl.PEAK_HBM_GBS, 4)}
    each = time_each(torch, spectral, max(100, min(K, 500)), R)
    log(f"[bench] spectral per launch: median {each['median']:.2f} us, min {each['min']:.2f} us")

    extra = {}
    if not args.no_expanded:
        for i in range(Wm):
            expanded(i % R)
        torch.cuda.synchronize()
        ms_e = timer(torch, expanded, K, R)
        each_e = time_each(torch, expanded, max(100, min(K, 500)), R)
        Fd = rl.dense_flops(w.N, w.C_in, w.C_out, w.G)
        Bd = rl.dense_bytes(w.N, w.C_in, w.C_out, w.G, eb)
        te = ms_e / 1e3
        tr, bd_ = rl.roof_time_s(Fd, Bd, peak_c)
        extra["expanded_baseline"] = {
            "ms_per_step": round(ms_e, 6), "tokens_per_s": w.N / te, "bound": bd_,
            "roof_frac": round(tr / te, 4), "mfma_frac": round(Fd / te / 1e12 / peak_c, 4),
            "hbm_frac": round(Bd / te / 1e9 / rl.PEAK_HBM_GBS, 4), "effective_tflops": round(Fd / te / 1e12, 2),
            "per_launch_us": each_e}
        extra["speedup_vs_expanded"] = round(ms_e / ms, 3)
        log(f"[bench] expanded: {ms_e * 1e3:.2f} us/step  speedup {ms_e / ms:.2f}x")
        if w.group == "cyclic":
            # context only, never the baseline: the same unrolled product through torch's F.linear
            # (the vendor GEMM library), the comparator the page measures against
            E = eq.export_expanded_weight(h)
            b_exp = bd.repeat_interleave(w.G)
            xf = [t.view(w.N, w.C_in * w.G) for t in xs]

            def torch_linear(i):
                torch.nn.functional.linear(xf[i], E, b_exp)

            # eager launches (a library GEMM is kept out of graph capture: its internal memsets are
            # not checked here for replay safety)
            try:
                for i in range(Wm):
                    torch_linear(i % R)
                torch.cuda.synchronize()
                ms_t = time_eager(torch, torch_linear, K, R)
                extra["torch_linear_context"] = {"ms_per_step": round(ms_t, 6), "tokens_per_s": w.N / (ms_t / 1e3),
                                                 "spectral_speedup": round(ms_t / ms, 3),
                                                 "timing": "eager launches"}
                log(f"[bench] torch F.linear on the unrolled weight (context): {ms_t * 1e3:.2f} us/step")
            except RuntimeError as e:  # context only: never fail the bench over it
                extra["torch_linear_context"] = {"error": str(e)[:200]}
            del E, b_exp, xf
    if args.backward:
        # the gradients of the same layer: dx on the forward kernels (transposed, group-reversed W),
        # dW and db by the frequency-domain products over tokens; dy is a seeded upstream gradient
        dy0 = make_grad(w.G, w.C_out, w.N, w.dtype, seed=0).to(dev)
        dys = [dy0] + [dy0.clone() for _ in range(R - 1)]
        dxs = [torch.empty_like(xd0) for _ in range(R)]
        ws = torch.empty((max(1, eq.backward_weights_workspace(h, w.N)),), dtype=torch.uint8, device=dev)
        dW = torch.empty((w.C_out, w.C_in, w.G), dtype=torch.float32, device=dev)
        db = torch.empty((w.C_out,), dtype=torch.float32, device=dev)
        lib = eq.load_library()
        import ctypes

        def bwd_data(i):
            eq.backward_data(h, dys[i], dxs[i])

        def bwd_weights(i):
            st = lib.eqlin_backward_weights(ctypes.c_void_p(h.ptr), ctypes.c_void_p(xs[i].data_ptr()),
                                            ctypes.c_void_p(dys[i].data_ptr()), ctypes.c_void_p(dW.data_ptr()),
                                            ctypes.c_void_p(db.data_ptr()), w.N, ctypes.c_void_p(ws.data_ptr()),
                                            ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if st != 0:
                raise RuntimeError(f"eqlin_backward_weights: {eq.status_string(st)}")

        res = {}
        for name, fn, Bk in (("data", bwd_data, B),
                             ("weights", bwd_weights,
                              w.N * (w.C_in + w.C_out) * w.G * eb + w.C_out * w.C_in * w.G * 4 + w.C_out * 4)):
            for i in range(Wm):
                fn(i % R)
            torch.cuda.synchronize()
            ms_b = timer(torch, fn, K, R)
            tb = ms_b / 1e3
            res[name] = {"ms_per_step": round(ms_b, 6), "tokens_per_s": w.N / tb,
                         "useful_tflops": round(F / tb / 1e12, 2), "mfma_frac": round(F / tb / 1e12 / peak_c, 4),
                         "algorithmic_bytes": Bk, "hbm_frac": round(Bk / tb / 1e9 / rl.PEAK_HBM_GBS, 4)}
            log(f"[bench] backward {name}: {ms_b * 1e3:.2f} us/step")
        res["kernels"] = h.describe().split("|")[3:]
        extra["backward"] = res
    if args.block:
        extra["block"] = bench_block(torch, eq, rl, timer, dev, K, Wm, not args.no_expanded)
    extra["effective_tflops"] = round(rl.dense_flops(w.N, w.C_in, w.C_out, w.G) / t / 1e12, 2)
    extra["useful_tflops"] = round(F / t / 1e12, 2)
    extra["per_launch_us"] = each

    line = {
        "metric": METRIC, "value": w.N / t, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded Gaussian x, W, b; see fourier_domain_linear_amd/workloads.py)",
        "config": {"workload": w.name, "group": w.group, "G": w.G, "C_in": w.C_in, "C_out": w.C_out, "tokens": w.N,
                   "timing": ("eager launches" if args.no_graph else "one HIP graph of K launches")
                   + f", {R} rotating buffer sets"},
        "roofline": roof,
    }
    line.update(extra)
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host cores ...")
        line["cpu_baseline"] = cpu_baseline(w, x, W, b)
    out = json.dumps(line)
    print(out, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(out + "\n")


if __name__ == "__main__":
    main()
