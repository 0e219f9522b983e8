"""Build libeqlin.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m fourier_domain_linear_amd.build          # compile every source, link the library

Objects go to fourier_domain_linear_amd/_build/, the library to fourier_domain_linear_amd/libeqlin.so.
Sources are compiled in parallel (one hipcc per file). Packed fp32 vector instructions are disabled
on the device side (-target-feature -packed-fp32-ops); the host pass warns that it does not know
the feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libeqlin.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]
# Per-file device flags. fwd_res8.hip: matrix-core results in ordinary vector registers (the weight ring
# and plane operands, which loads can fill directly, take the accumulator registers instead), so the
# epilogue reads its eleven accumulators without a copy per value and no register is spilled.
FILE_FLAGS = {"fwd_res8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
SOURCES = ["eqlin_api.cpp", "prepare.hip", "fwd_bf16.hip", "fwd_big.hip", "fwd_res.hip", "fwd_res8.hip", "fwd_f32.hip", "bwd.hip", "conv.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *CXXFLAGS, *FILE_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
