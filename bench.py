#!/usr/bin/env python3
"""Benchmark of the EQ-Linear spectral forward on one MI355X.

A step is one eqlin_forward over one batch of the workload (the whole hot path: load, group DFT,
per-frequency products, inverse DFT + bias, store -- one fused kernel). Default workload: the largest
configured one, p8 (G = 8), C_in = 256 -> C_out = 1024, N = 64x14x14 = 12544 tokens, bf16 in/out,
synthetic seeded inputs (matrix-core bound). The line also carries a table ("configs") with every
configured workload's spectral and expanded times, roofline fractions and speedup.

Timing. Inputs are resident in HBM before the timed region. W warmup steps run eagerly; then K steps
are captured into one HIP graph (so the ~10 us kernels are not bounded by host launch latency) and
replayed untimed (one replay at a time) for at least SETTLE_S = 0.25 s and then once timed, between
HIP events on the launch stream, with torch.cuda.synchronize() on both sides. The W warm-up steps are
likewise followed by more of the same launches until SETTLE_S has passed: the GPU's clock rises over
tens of milliseconds of sustained work, and a few steps timed right after a short warm-up (or after the
idle gap of the capture) run well below it. The K steps rotate over R buffer sets totalling >= 1 GiB,
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


def load_traffic(workload: str, kernel_desc: str | None = None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the kernel
    family the plan runs (kernel_desc: the plan's forward kernel name) and on its current sources (else
    None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from fourier_domain_linear_amd.profiling import KERNEL_SOURCES, family_of_plan, kernel_source_hash

    rec_family = next((f for f in sorted(KERNEL_SOURCES, key=len, reverse=True) if rec.get("kernel", "").startswith(f)),
                      None)
    if kernel_desc is not None and rec_family != family_of_plan(kernel_desc):
        log(f"[bench] {path} was taken on another kernel ({rec.get('kernel')}): traffic = null")
        return None
    if rec.get("source_sha256") != kernel_source_hash(rec.get("sources")):
        log(f"[bench] {path} was taken on other kernel sources: traffic = null")
        return None
    return rec.get("traffic_bytes_per_launch")


# The warm-up runs for at least this long: the GPU's clock rises over tens of milliseconds of sustained
# work, and a few steps timed right after a short warm-up run below the steady clock (measured: 148 us
# per step at 20 steps after 5 warm-up launches against 113-115 us at 500 after 50, headline workload).
SETTLE_S = 0.25


def warm_up(torch, launch, Wm: int, R: int):
    """The W warm-up launches (launch(i) uses buffer set i % R), then more of the same, in synchronised
    rounds of max(W, 64), until at least SETTLE_S seconds have passed since the first."""
    t0 = time.perf_counter()
    for i in range(Wm):
        launch(i % R)
    torch.cuda.synchronize()
    n = max(Wm, 64)
    while time.perf_counter() - t0 < SETTLE_S:
        for i in range(n):
            launch(i % R)
        torch.cuda.synchronize()


def time_graph(torch, launch, K: int, R: int):
    """Capture K launches (launch(i) uses buffer set i % R) into one graph; replay it untimed, one
    replay at a time, until at least SETTLE_S seconds have passed (the capture leaves the GPU idle long
    enough for its clock to drop again), then once timed. Returns ms per launch."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            launch(i % R)
    t0 = time.perf_counter()
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= SETTLE_S:
            break
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


def bench_backward(torch, eq, rl, w, st, dev, K: int, Wm: int, timer, with_expanded: bool):
    """Time the gradients of the headline layer: eqlin_backward_data (dx on the forward kernels over the
    transposed, group-reversed weight) and eqlin_backward_weights (dW, db by frequency-domain products
    over tokens); dy is a seeded upstream gradient."""
    import ctypes

    from fourier_domain_linear_amd.workloads import make_grad

    h, xs, R, F, B, peak_c = st["h"], st["xs"], st["R"], st["F"], st["B"], st["peak_c"]
    eb = w.elem_bytes
    dy0 = make_grad(w.G, w.C_out, w.N, w.dtype, seed=0).to(dev)
    dys = [dy0] + [dy0.clone() for _ in range(R - 1)]
    dxs = [torch.empty_like(xs[0]) for _ in range(R)]
    ws = torch.empty((max(1, eq.backward_weights_workspace(h, w.N)),), dtype=torch.uint8, device=dev)
    dW = torch.empty((w.C_out, w.C_in, w.G), dtype=torch.float32, device=dev)
    db = torch.empty((w.C_out,), dtype=torch.float32, device=dev)
    lib = eq.load_library()

    def bwd_data(i):
        eq.backward_data(h, dys[i], dxs[i])

    def bwd_weights(i):
        st_ = lib.eqlin_backward_weights(ctypes.c_void_p(h.ptr), ctypes.c_void_p(xs[i].data_ptr()),
                                         ctypes.c_void_p(dys[i].data_ptr()), ctypes.c_void_p(dW.data_ptr()),
                                         ctypes.c_void_p(db.data_ptr()), w.N, ctypes.c_void_p(ws.data_ptr()),
                                         ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st_ != 0:
            raise RuntimeError(f"eqlin_backward_weights: {eq.status_string(st_)}")

    res = {}
    for name, fn, Bk in (("data", bwd_data, B),
                         ("weights", bwd_weights,
                          w.N * (w.C_in + w.C_out) * w.G * eb + w.C_out * w.C_in * w.G * 4 + w.C_out * 4)):
        warm_up(torch, fn, Wm, R)
        ms_b = timer(torch, fn, K, R)
        tb = ms_b / 1e3
        res[name] = {"us_per_step": round(ms_b * 1e3, 3), "tokens_per_s": w.N / tb,
                     "useful_tflops": round(F / tb / 1e12, 2), "mfma_frac": round(F / tb / 1e12 / peak_c, 4),
                     "algorithmic_bytes": Bk, "hbm_frac": round(Bk / tb / 1e9 / rl.PEAK_HBM_GBS, 4)}
        log(f"[bench] backward {name}: {ms_b * 1e3:.2f} us/step")
    res["kernels"] = h.describe().split("|")[3:]
    if with_expanded and w.group == "cyclic":
        # the naive layer's gradients (replicate the weight, multiply densely): dx = dy E on the
        # hand-written G = 1 kernels over E^T, and dE = dy^T x through torch's matrix product (the vendor
        # GEMM, as autograd computes a dense layer's weight gradient) folded back onto W along the
        # circulant diagonals, dW[o, i, d] = sum_h dE[o G + h, i G + (h - d) mod G]
        dxe = [torch.empty_like(xs[0]) for _ in range(R)]

        def bwd_data_exp(i):
            eq.backward_data_expanded(h, dys[i], dxe[i])

        G, Co, Ci = w.G, w.C_out, w.C_in
        nset = min(R, 3)
        dyT = [dys[i].view(w.N, Co * G).t().contiguous() for i in range(nset)]  # outside the timed region
        xf = [xs[i].view(w.N, Ci * G) for i in range(nset)]
        hh = torch.arange(G, device=dev)
        index = ((hh[:, None] - hh[None, :]) % G).expand(Co, Ci, G, G)  # [o, i, h, d] -> g = (h - d) mod G

        def bwd_weights_naive(i):
            dE = torch.mm(dyT[i % nset], xf[i % nset])  # [Co G, Ci G]
            torch.gather(dE.view(Co, G, Ci, G).permute(0, 2, 1, 3), 3, index).sum(dim=2)

        exp = {}
        for name, fn, timer_ in (("data_expanded", bwd_data_exp, timer), ("weights_naive", bwd_weights_naive, time_eager)):
            try:
                warm_up(torch, fn, Wm, R)
                exp[name] = {"us_per_step": round(timer_(torch, fn, K, R) * 1e3, 3)}
                log(f"[bench] backward {name}: {exp[name]['us_per_step']:.2f} us/step")
            except RuntimeError as e:  # the torch leg is a comparator: report, never fail the bench
                exp[name] = {"error": str(e)[:200]}
        exp["weights_naive"]["timing"] = "eager launches: torch.mm (dy^T x) + gather/sum fold"
        exp["data_expanded"]["kernel"] = "hand-written G = 1 product over E^T (eqlin_backward_data_expanded)"
        res["expanded"] = exp
        if "us_per_step" in exp["data_expanded"]:
            res["data"]["speedup_vs_expanded"] = round(exp["data_expanded"]["us_per_step"] / res["data"]["us_per_step"], 3)
        if "us_per_step" in exp["weights_naive"]:
            res["weights"]["speedup_vs_naive"] = round(exp["weights_naive"]["us_per_step"] / res["weights"]["us_per_step"], 3)
        if "us_per_step" in exp["data_expanded"] and "us_per_step" in exp["weights_naive"]:
            tot_s = res["data"]["us_per_step"] + res["weights"]["us_per_step"]
            tot_e = exp["data_expanded"]["us_per_step"] + exp["weights_naive"]["us_per_step"]
            res["speedup_vs_expanded"] = round(tot_e / tot_s, 3)
            log(f"[bench] backward (dx + dW): spectral {tot_s:.1f} us, naive {tot_e:.1f} us, {tot_e / tot_s:.2f}x")
    return res


def bench_conv(torch, eq, rl, timer, dev, K: int, Wm: int):
    """Time the p4 group convolution (eqlin_conv_forward: the EQ-Linear layer over the gathered channels,
    gathered while x is loaded) and its unrolled comparator (eqlin_conv_forward_expanded), plus torch's
    conv2d on the fully unrolled filter bank as context (the plain way to run a group convolution)."""
    from fourier_domain_linear_amd.workloads import CONV_WORKLOAD as cw, make_conv_inputs

    Ci, Co, k, N = cw.C_in, cw.C_out, cw.k, cw.N
    log(f"[bench] conv {cw.name}: p4 {k}x{k} C_in={Ci} C_out={Co} {cw.B}x{cw.H}x{cw.W} {cw.dtype}")
    x, psi, b = make_conv_inputs(Ci, Co, k, cw.B, cw.H, cw.W, cw.dtype, seed=0)
    set_bytes = N * (Ci + Co) * 4 * 2
    R = max(3, math.ceil((1 << 30) / set_bytes))
    x0 = x.to(dev)
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    ys = [torch.empty((cw.B, cw.H, cw.W, Co, 4), dtype=cw.torch_dtype, device=dev) for _ in range(R)]
    h = eq.prepare_conv_weights(psi.to(dev), expanded=True)
    bd = b.to(dev)
    torch.cuda.synchronize()
    log(f"[bench] {h.describe()}")
    Cg = Ci * k * k  # gathered channels
    F = rl.spectral_flops(N, Cg, Co, 4)
    Fd = rl.dense_flops(N, Cg, Co, 4)
    B = rl.spectral_bytes(N, Ci, Co, 4, 2) + (Cg - Ci) * Co * 4 * 2  # x, y, the gathered layer's planes, bias
    res = {"workload": cw.name, "k": k, "C_in": Ci, "C_out": Co, "images": [cw.B, cw.H, cw.W], "tokens": N,
           "gathered_channels": Cg, "kernels": h.describe(), "algorithmic_flops": F, "algorithmic_bytes": B}
    for name, fn, flops in (("spectral", lambda i: eq.conv_forward(h, xs[i], bd, ys[i]), F),
                            ("expanded", lambda i: eq.conv_forward_expanded(h, xs[i], bd, ys[i]), Fd)):
        warm_up(torch, fn, Wm, R)
        ms = timer(torch, fn, K, R)
        t = ms / 1e3
        res[name] = {"us_per_step": round(ms * 1e3, 3), "tokens_per_s": N / t, "tflops": round(flops / t / 1e12, 2),
                     "mfma_frac": round(flops / t / 1e12 / rl.PEAK_BF16_TFLOPS, 4),
                     "hbm_frac": round(B / t / 1e9 / rl.PEAK_HBM_GBS, 4)}
        log(f"[bench] conv {name}: {ms * 1e3:.2f} us/step")
    tr, bound = rl.roof_time_s(F, B, rl.PEAK_BF16_TFLOPS)
    res["bound"] = bound
    res["frac"] = round(tr / (res["spectral"]["us_per_step"] / 1e6), 4)
    # HBM bytes per launch of the spectral kernel, from the committed counter summary (null when it
    # was taken on other kernel sources): the gather reads each pixel's row k^2 times from the caches
    res["traffic"] = load_traffic(cw.name)
    res["speedup_vs_expanded"] = round(res["expanded"]["us_per_step"] / res["spectral"]["us_per_step"], 3)
    # context: torch conv2d (the vendor convolution library) on the unrolled filter bank
    # Wfull[(o, h), (i, g)] = psi[o, i, (h - g) mod 4] turned h quarter turns, input in NCHW
    try:
        Wf = torch.empty((Co, 4, Ci, 4, k, k), dtype=torch.float32)
        pf = psi.float()
        for hh in range(4):
            for g in range(4):
                Wf[:, hh, :, g] = torch.rot90(pf[:, :, (hh - g) % 4], hh, dims=(2, 3))
        Wf = Wf.reshape(Co * 4, Ci * 4, k, k).to(cw.torch_dtype).to(dev)
        xn = [v.reshape(cw.B, cw.H, cw.W, Ci * 4).permute(0, 3, 1, 2).contiguous() for v in xs[:2]]
        bf = bd.repeat_interleave(4)

        def torch_conv(i):
            torch.nn.functional.conv2d(xn[i % 2], Wf, bf, padding=k // 2)

        warm_up(torch, torch_conv, Wm, R)
        ms_t = time_eager(torch, torch_conv, K, 2)
        res["torch_conv2d_context"] = {"us_per_step": round(ms_t * 1e3, 3),
                                       "spectral_speedup": round(ms_t * 1e3 / res["spectral"]["us_per_step"], 3),
                                       "timing": "eager launches, NCHW input, 2 buffer sets"}
        log(f"[bench] torch conv2d on the unrolled filters (context): {ms_t * 1e3:.2f} us/step")
    except RuntimeError as e:  # context only
        res["torch_conv2d_context"] = {"error": str(e)[:200]}
    return res


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
        warm_up(torch, fn, Wm, R)
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


def measure_forward(torch, eq, rl, w, dev, K: int, Wm: int, timer, with_expanded: bool = True,
                    with_torch: bool = False, with_each: bool = True, backward: bool = False, inputs=None):
    """Time eqlin_forward (and eqlin_forward_expanded) on workload w's seeded inputs (or `inputs`, an
    (x, W, b) of w's shape), resident in HBM and rotated over >= 1 GiB of buffer sets. Returns (record,
    state) where record holds the figures and state the tensors and handle a caller may reuse."""
    x, W, b = inputs if inputs is not None else workload_inputs_for(w)
    eb = w.elem_bytes
    set_bytes = w.N * (w.C_in + w.C_out) * w.G * eb
    R = max(3, math.ceil((1 << 30) / set_bytes))
    xd0 = x.to(dev)
    xs = [xd0] + [xd0.clone() for _ in range(R - 1)]
    ys = [torch.empty((w.N, w.C_out, w.G), dtype=w.torch_dtype, device=dev) for _ in range(R)]
    bd = b.to(dev)
    h = eq.prepare_weights(W.to(dev), expanded=with_expanded, backward=backward, group=w.group)
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: {h.describe()}  rotating buffer sets: {R} ({R * set_bytes / 2**20:.0f} MiB)")

    def spectral(i):
        eq.forward(h, xs[i], bd, ys[i])

    def expanded(i):
        eq.forward_expanded(h, xs[i], bd, ys[i])

    warm_up(torch, spectral, Wm, R)
    ms = timer(torch, spectral, K, R)
    log(f"[bench] {w.name} spectral: {ms * 1e3:.2f} us/step")
    F = rl.spectral_flops(w.N, w.C_in, w.C_out, w.G, w.group)
    B = rl.spectral_bytes(w.N, w.C_in, w.C_out, w.G, eb)
    # fp16 matrix cores have the bf16 dense peak on this chip (2.5 PFLOP/s)
    peak_c = rl.PEAK_BF16_TFLOPS if w.dtype in ("bf16", "f16") else rl.PEAK_FP32_TFLOPS
    _, bound = rl.roof_time_s(F, B, peak_c)
    t = ms / 1e3
    rec = {"workload": w.name, "us_per_step": round(ms * 1e3, 3), "tokens_per_s": w.N / t, "bound": bound,
           "frac": round((B / t / 1e9 / rl.PEAK_HBM_GBS) if bound == "hbm" else (F / t / 1e12 / peak_c), 4),
           "mfma_frac": round(F / t / 1e12 / peak_c, 4), "hbm_frac": round(B / t / 1e9 / rl.PEAK_HBM_GBS, 4),
           "useful_tflops": round(F / t / 1e12, 2),
           "effective_tflops": round(rl.dense_flops(w.N, w.C_in, w.C_out, w.G) / t / 1e12, 2),
           "kernel": h.describe().split("|")[1].strip().removeprefix("forward: ")}
    state = {"x": x, "W": W, "b": b, "xs": xs, "ys": ys, "bd": bd, "h": h, "R": R, "ms": ms, "F": F, "B": B,
             "peak_c": peak_c, "bound": bound, "spectral": spectral}
    if with_each:
        rec["per_launch_us"] = time_each(torch, spectral, max(100, min(K, 500)), R)
        log(f"[bench] {w.name} spectral per launch: median {rec['per_launch_us']['median']:.2f} us, "
            f"min {rec['per_launch_us']['min']:.2f} us")
    if with_expanded:
        warm_up(torch, expanded, Wm, R)
        ms_e = timer(torch, expanded, K, R)
        Fd = rl.dense_flops(w.N, w.C_in, w.C_out, w.G)
        Bd = rl.dense_bytes(w.N, w.C_in, w.C_out, w.G, eb)
        te = ms_e / 1e3
        tr, bd_ = rl.roof_time_s(Fd, Bd, peak_c)
        exp = {"us_per_step": round(ms_e * 1e3, 3), "tokens_per_s": w.N / te, "bound": bd_,
               "roof_frac": round(tr / te, 4), "mfma_frac": round(Fd / te / 1e12 / peak_c, 4),
               "hbm_frac": round(Bd / te / 1e9 / rl.PEAK_HBM_GBS, 4), "effective_tflops": round(Fd / te / 1e12, 2),
               "kernel": h.describe().split("|")[2].strip().removeprefix("expanded: ")}
        if with_each:
            exp["per_launch_us"] = time_each(torch, expanded, max(100, min(K, 500)), R)
        rec["expanded"] = exp
        rec["speedup_vs_expanded"] = round(ms_e / ms, 3)
        log(f"[bench] {w.name} expanded: {ms_e * 1e3:.2f} us/step  speedup {ms_e / ms:.2f}x")
        if with_torch and w.group == "cyclic":
            # context only, never the baseline: the same unrolled product through torch's F.linear
            # (the vendor GEMM library), the comparator the page measures against
            E = eq.export_expanded_weight(h)
            b_exp = bd.repeat_interleave(w.G)
            xf = [v.view(w.N, w.C_in * w.G) for v in xs]

            def torch_linear(i):
                torch.nn.functional.linear(xf[i], E, b_exp)

            # eager launches (a library GEMM is kept out of graph capture: its internal memsets are
            # not checked here for replay safety)
            try:
                warm_up(torch, torch_linear, Wm, R)
                ms_t = time_eager(torch, torch_linear, K, R)
                rec["torch_linear_context"] = {"us_per_step": round(ms_t * 1e3, 3),
                                               "tokens_per_s": w.N / (ms_t / 1e3),
                                               "spectral_speedup": round(ms_t / ms, 3), "timing": "eager launches"}
                log(f"[bench] torch F.linear on the unrolled weight (context): {ms_t * 1e3:.2f} us/step")
            except RuntimeError as e:  # context only: never fail the bench over it
                rec["torch_linear_context"] = {"error": str(e)[:200]}
            del E, b_exp, xf
    return rec, state


def bench_shards(torch, eq, rl, timer, dev, K: int, Wm: int, parts):
    """The kernel at one shard's shape: each bf16 workload's spectral forward on the first N/P tokens of
    its inputs, for P in `parts`, timed like the headline on this one GPU. The layer is token-parallel
    with no communication, so a shard of P is this launch on its own device; what the table shows is how
    the kernel's efficiency holds up as the per-device token count falls (launch cost, wave
    quantisation). No figure for several devices is derived from it."""
    import dataclasses

    from fourier_domain_linear_amd.workloads import WORKLOADS

    out = {}
    for wf in WORKLOADS:
        if wf.dtype != "bf16":
            continue
        x, W, b = workload_inputs_for(wf)
        per = {}
        for P in parts:
            n = wf.N // P
            ws = dataclasses.replace(wf, name=f"{wf.name}_shard_1_of_{P}", N=n)
            r, _ = measure_forward(torch, eq, rl, ws, dev, K, Wm, timer, with_expanded=False, with_each=False,
                                   inputs=(x[:n].contiguous(), W, b))
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            per[str(P)] = {"tokens": n, "us_per_step": r["us_per_step"], "tokens_per_s": r["tokens_per_s"],
                           "bound": r["bound"], "frac": r["frac"], "kernel": r["kernel"]}
        out[wf.name] = per
    return out


_INPUT_CACHE = {}


def workload_inputs_for(w):
    from fourier_domain_linear_amd.workloads import workload_inputs

    if w.name not in _INPUT_CACHE:
        _INPUT_CACHE.clear()
        _INPUT_CACHE[w.name] = workload_inputs(w, seed=0)
    return _INPUT_CACHE[w.name]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None,
                    help="workload name (default: the largest, p8 256->1024 channels, 12544 tokens)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-expanded", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload table (every configured workload, spectral and expanded)")
    ap.add_argument("--config-steps", type=int, default=200, help="timed steps per workload of the table")
    ap.add_argument("--json-out", default=None, help="also write the JSON line to this file")
    ap.add_argument("--backward", action="store_true",
                    help="also time eqlin_backward_data and eqlin_backward_weights, and the same gradients "
                         "through the unrolled weight (reported under 'backward')")
    ap.add_argument("--block", action="store_true",
                    help="also time the transformer MLP block EQ-Linear(C->4C), GELU, EQ-Linear(4C->C) at the "
                         "p4 192-channel shape, spectral and expanded (reported under 'block')")
    ap.add_argument("--conv", action="store_true",
                    help="also time the p4 3x3 group convolution, spectral and expanded (reported under 'conv')")
    ap.add_argument("--shards", default=None, metavar="P,P,...",
                    help="also time each bf16 workload's kernel on one shard of N/P tokens (one GPU)")
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
    from fourier_domain_linear_amd.workloads import BENCH_WORKLOAD, BY_NAME, WORKLOADS

    w = BY_NAME[args.workload] if args.workload else BENCH_WORKLOAD
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    eq.load_library()

    K, Wm = args.steps, args.warmup
    timer = time_eager if args.no_graph else time_graph
    log(f"[bench] workload {w.name}: G={w.G} C_in={w.C_in} C_out={w.C_out} N={w.N} {w.dtype} ({w.group})")
    rec, st = measure_forward(torch, eq, rl, w, dev, K, Wm, timer, with_expanded=not args.no_expanded,
                              with_torch=True, with_each=True, backward=args.backward)
    ms, F, B, peak_c, bound = st["ms"], st["F"], st["B"], st["peak_c"], st["bound"]
    t = ms / 1e3
    if bound == "hbm":
        achieved, peak, unit = B / t / 1e9, rl.PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = F / t / 1e12, peak_c, "TFLOP/s"
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": load_traffic(w.name, rec["kernel"]),
            "kernel": rec["kernel"] + " (one launch per step)",
            "algorithmic_bytes_per_launch": B, "algorithmic_flops_per_launch": F,
            "mfma_frac": rec["mfma_frac"], "hbm_frac": rec["hbm_frac"]}

    extra = {}
    if "expanded" in rec:
        e = rec["expanded"]
        extra["expanded_baseline"] = {k: v for k, v in e.items()}
        extra["expanded_baseline"]["ms_per_step"] = round(e["us_per_step"] / 1e3, 6)
        extra["speedup_vs_expanded"] = rec["speedup_vs_expanded"]
    if "torch_linear_context" in rec:
        extra["torch_linear_context"] = rec["torch_linear_context"]
    if args.backward:
        extra["backward"] = bench_backward(torch, eq, rl, w, st, dev, K, Wm, timer, not args.no_expanded)
    if args.block:
        extra["block"] = bench_block(torch, eq, rl, timer, dev, K, Wm, not args.no_expanded)
    if args.conv:
        extra["conv"] = bench_conv(torch, eq, rl, timer, dev, K, Wm)
    if args.shards:
        parts = [int(v) for v in args.shards.split(",") if v]
        if any(P < 1 for P in parts):
            raise SystemExit("--shards: each P must be >= 1")
        extra["shards"] = bench_shards(torch, eq, rl, timer, dev, min(K, args.config_steps),
                                       min(Wm, args.config_steps), parts)
    extra["effective_tflops"] = rec["effective_tflops"]
    extra["useful_tflops"] = rec["useful_tflops"]
    extra["per_launch_us"] = rec["per_launch_us"]
    x, W, b = st["x"], st["W"], st["b"]
    del st
    if not args.no_configs:
        # every configured workload (the headline's figures reused), spectral and expanded
        table = {}
        for wc in WORKLOADS:
            if wc.name == w.name:
                r = {k: v for k, v in rec.items() if k not in ("per_launch_us", "torch_linear_context")}
                if "expanded" in r:
                    r["expanded"] = {k: v for k, v in r["expanded"].items() if k != "per_launch_us"}
            else:
                r, _ = measure_forward(torch, eq, rl, wc, dev, min(K, args.config_steps),
                                       min(Wm, args.config_steps), timer, with_expanded=not args.no_expanded,
                                       with_each=False)
                torch.cuda.synchronize()
                torch.cuda.empty_cache()
            table[wc.name] = r
        extra["configs"] = table

    line = {
        "metric": METRIC, "value": w.N / t, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded Gaussian x, W, b; see fourier_domain_linear_amd/workloads.py)",
        "config": {"workload": w.name, "group": w.group, "G": w.G, "C_in": w.C_in, "C_out": w.C_out, "tokens": w.N,
                   "timing": ("eager launches" if args.no_graph else "one HIP graph of K launches")
                   + f" after >= {SETTLE_S} s of warm-up (launches, then untimed replays), rotating buffer sets"
                   + " over >= 1 GiB"},
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
