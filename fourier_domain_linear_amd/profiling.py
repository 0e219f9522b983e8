"""Summaries of rocprofv3 output for the profiles/ directory.

    # kernel durations (rocprofv3 --kernel-trace --stats -f csv ...)
    python -m fourier_domain_linear_amd.profiling stats DIR --cmd "<the rocprofv3 command>" --out FILE.txt

    # HBM traffic per launch from two counter runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch),
    # each scaled by what the same counter reads for a plain device copy of known size
    python -m fourier_domain_linear_amd.profiling traffic --kernel k_stream \
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes B \
        --workload NAME --cmd "..." --out profiles/traffic_NAME.json [--family k_conv]

    # matrix-core utilisation from one counter run (SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA
    # SQ_INSTS_VALU GRBM_GUI_ACTIVE)
    python -m fourier_domain_linear_amd.profiling mfma DIR --kernel k_p8 --workload NAME \
        --cmd "..." --out profiles/mfma_NAME.txt

DIR is a rocprofv3 output directory (-d); the CSV files are found by name inside it.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_COMMON = ["fourier_domain_linear_amd/csrc/device_common.h", "fourier_domain_linear_amd/csrc/dft.h",
           "fourier_domain_linear_amd/csrc/act.h"]
# the sources each forward kernel family is built from (a counter summary is valid only for these)
KERNEL_SOURCES = {
    "k_stream": ["fourier_domain_linear_amd/csrc/fwd_bf16.hip"] + _COMMON,
    "k_big": ["fourier_domain_linear_amd/csrc/fwd_big.hip"] + _COMMON,
    "k_p8": ["fourier_domain_linear_amd/csrc/fwd_big.hip"] + _COMMON,
    "k_conv": ["fourier_domain_linear_amd/csrc/fwd_big.hip", "fourier_domain_linear_amd/csrc/conv.hip"] + _COMMON,
    "k_res": ["fourier_domain_linear_amd/csrc/fwd_res.hip"] + _COMMON,
    "k_res8": ["fourier_domain_linear_amd/csrc/fwd_res8.hip"] + _COMMON,
}


def family_of_plan(desc: str) -> str:
    """The kernel family a plan's forward runs, from its name in eqlin_describe's forward field."""
    if "resident" in desc:
        return "k_res8" if ("G=8" in desc or "D4" in desc) else "k_res"
    if "stream" in desc:
        return "k_stream"
    if "gathered" in desc:
        return "k_conv"
    if "big" in desc:
        return "k_p8" if ("G=8" in desc or "D4" in desc) else "k_big"
    return "other"


def sources_for(kernel: str) -> list:
    """The source list of the kernel family whose name starts `kernel` (e.g. "k_p8<false, ...>")."""
    for fam in sorted(KERNEL_SOURCES, key=len, reverse=True):
        if kernel.startswith(fam):
            return KERNEL_SOURCES[fam]
    raise ValueError(f"unknown kernel family for {kernel!r}")


def kernel_source_hash(sources: list | None = None) -> str:
    """sha256 over a kernel family's sources (default: the stream kernel's)."""
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES["k_stream"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _find(d: str, pattern: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return hits[0]


def kernel_stats(d: str):
    """Rows of the rocprofv3 kernel statistics CSV: (name, calls, avg_ns, min_ns, max_ns, total_ns, pct)."""
    rows = []
    with open(_find(d, "*kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                         float(r["MaxNs"]), float(r["TotalDurationNs"]), float(r["Percentage"])))
    return rows


def counter_per_dispatch(d: str, kernel: str, counter: str):
    """Values of `counter` summed over its hardware instances, one per dispatch of kernels whose
    name contains `kernel`."""
    per = collections.defaultdict(float)
    with open(_find(d, "*counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
                per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise ValueError(f"no {counter} samples for kernels matching {kernel!r} in {d}")
    return list(per.values())


def dispatches(d: str, kernel: str):
    """Per dispatch of kernels whose name contains `kernel`: (kernel name, duration in ns, {counter:
    value summed over its hardware instances})."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    meta = {}
    with open(_find(d, "*counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"]:
                per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
                meta[r["Dispatch_Id"]] = (r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if not per:
        raise ValueError(f"no counter samples for kernels matching {kernel!r} in {d}")
    return [(meta[k][0], meta[k][1], dict(v)) for k, v in per.items()]


def _avg(v):
    return sum(v) / len(v)


def cmd_stats(a):
    rows = kernel_stats(a.dir)
    lines = [f"# rocprofv3 kernel statistics", f"# command: {a.cmd}", "",
             f"{'kernel':<90} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}"]
    for name, calls, avg, mn, mx, tot, pct in sorted(rows, key=lambda r: -r[5]):
        lines.append(f"{name[:90]:<90} {calls:>6} {avg / 1e3:>9.3f} {mn / 1e3:>9.3f} {mx / 1e3:>9.3f} {pct:>6.2f}")
    if a.bench_json:
        # the profiled bench.py run's own figures (graph-timed under the profiler, same process)
        with open(a.bench_json) as f:
            line = json.load(f)
        lines += ["", f"# the profiled run's bench line: workload {line['config']['workload']}, "
                      f"{line['ms_per_step'] * 1e3:.3f} us per step graph-timed over {line['steps']} steps "
                      f"(the averages above also count the warm-up and per-launch eager launches)"]
        for name, rec in sorted((line.get("configs") or {}).items()):
            lines.append(f"#   {name}: {rec['us_per_step']:.3f} us per step ({rec['kernel']})")
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


def cmd_traffic(a):
    fetch = counter_per_dispatch(a.fetch, a.kernel, "FETCH_SIZE")
    write = counter_per_dispatch(a.write, a.kernel, "WRITE_SIZE")
    cfetch = counter_per_dispatch(a.copy_fetch, a.copy_kernel, "FETCH_SIZE")
    cwrite = counter_per_dispatch(a.copy_write, a.copy_kernel, "WRITE_SIZE")
    # the copy reads and writes copy_bytes each: bytes per KiB of counter reading
    f_scale = a.copy_bytes / _avg(cfetch)
    w_scale = a.copy_bytes / _avg(cwrite)
    rd, wr = _avg(fetch) * f_scale, _avg(write) * w_scale
    srcs = KERNEL_SOURCES[a.family] if a.family else sources_for(a.kernel)
    rec = {
        "workload": a.workload, "kernel": a.kernel, "sources": srcs, "source_sha256": kernel_source_hash(srcs),
        "fetch_kib_per_dispatch": _avg(fetch), "write_kib_per_dispatch": _avg(write),
        "copy_bytes": a.copy_bytes, "copy_fetch_kib": _avg(cfetch), "copy_write_kib": _avg(cwrite),
        "fetch_scale_bytes_per_kib": f_scale, "write_scale_bytes_per_kib": w_scale,
        "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
        "traffic_bytes_per_launch": rd + wr, "dispatches": [len(fetch), len(write)], "command": a.cmd,
    }
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def cmd_mfma(a):
    """Matrix-core busy fraction: SQ_VALU_MFMA_BUSY_CYCLES counts, summed over every SIMD, the cycles
    its matrix core is busy (32 per 32x32x16 and 16 per 16x16x32 bf16 instruction); GRBM_GUI_ACTIVE
    counts the busy cycles of each XCD's graphics engine over the dispatch (summed over the XCDs)."""
    from fourier_domain_linear_amd import roofline as rl
    from fourier_domain_linear_amd.workloads import BY_NAME

    rows = dispatches(a.dir, a.kernel)
    names = sorted({r[0] for r in rows})
    dur = _avg([r[1] for r in rows])
    c = {k: _avg([r[2].get(k, 0.0) for r in rows]) for k in
         ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE")}
    cyc = c["GRBM_GUI_ACTIVE"] / a.xcds
    busy_grbm = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (a.simds * cyc) if cyc else float("nan")
    busy_dur = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (a.simds * dur * a.clock_ghz)
    w = BY_NAME[a.workload]
    flop = rl.spectral_flops(w.N, w.C_in, w.C_out, w.G, w.group)
    issued = c["SQ_INSTS_MFMA"] * a.inst_flop
    lines = [
        "# matrix-core utilisation per launch (rocprofv3 --pmc, one pass)",
        f"# command: {a.cmd}",
        f"workload: {a.workload}",
        "kernel: " + " / ".join(names),
        f"dispatches averaged: {len(rows)}",
        f"duration (counters on), us: {dur / 1e3:.3f}",
        f"SQ_INSTS_MFMA: {c['SQ_INSTS_MFMA']:.0f}  (x {a.inst_flop} FLOP = {issued:.4g} issued;"
        f" useful {flop:.4g}, ratio {issued / flop:.4f})",
        f"SQ_VALU_MFMA_BUSY_CYCLES: {c['SQ_VALU_MFMA_BUSY_CYCLES']:.0f}",
        f"SQ_INSTS_VALU: {c['SQ_INSTS_VALU']:.0f}  ({c['SQ_INSTS_VALU'] / max(1.0, c['SQ_INSTS_MFMA']):.2f} per MFMA)",
        f"GRBM_GUI_ACTIVE: {c['GRBM_GUI_ACTIVE']:.0f}  ({cyc:.0f} per XCD over {a.xcds} XCDs: the engines' busy"
        f" window, dispatch set-up included)",
        f"matrix-core busy fraction, over the kernel duration at {a.clock_ghz} GHz: {busy_dur:.4f}",
        f"matrix-core busy fraction, over the GRBM_GUI_ACTIVE window: {busy_grbm:.4f}",
        f"useful TFLOP/s at the profiled duration: {flop / dur / 1e3:.1f}"
        f" ({flop / dur / 1e3 / rl.PEAK_BF16_TFLOPS:.4f} of the 2.5 PFLOP/s bf16 peak)",
    ]
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--cmd", required=True)
    s.add_argument("--bench-json", help="bench.py --json-out file of the profiled run")
    s.add_argument("--out")
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--family", choices=sorted(KERNEL_SOURCES), default=None,
                   help="the kernel family whose sources the record covers (default: by the name's prefix; "
                        "the gathered-load k_big instances are k_conv)")
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("--kernel", required=True)
    m.add_argument("--workload", required=True)
    m.add_argument("--simds", type=int, default=1024)
    m.add_argument("--xcds", type=int, default=8)
    m.add_argument("--clock-ghz", type=float, default=2.4)
    m.add_argument("--inst-flop", type=int, default=32768,
                   help="FLOP per matrix-core instruction (32x32x16: 32768, 16x16x32: 16384)")
    m.add_argument("--cmd", required=True)
    m.add_argument("--out")
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "mfma": cmd_mfma}[a.what](a)


if __name__ == "__main__":
    main()
