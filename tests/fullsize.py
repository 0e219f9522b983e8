"""Element-by-element comparison of full-size GPU results with an fp64 oracle, in token chunks.

At the workloads' full token counts the whole result is compared: the oracle is run over chunks of
tokens (bounding host memory: at most one chunk of the fp64 reference is alive), each chunk is set
against the same rows of every GPU result, and the relative Frobenius error and the maximum
absolute error are accumulated over all tokens (sums of squares and a running maximum).
"""
from __future__ import annotations

import math

import numpy as np
import torch


class Errors:
    """Running relative-Frobenius and max-abs errors of one GPU result against a reference."""

    def __init__(self, label: str):
        self.label = label
        self.ss_diff = 0.0
        self.ss_ref = 0.0
        self.max_abs = 0.0
        self.max_ref_rms = 0.0
        self.finite = True
        self.count = 0

    def add(self, got: np.ndarray, ref: np.ndarray):
        if got.shape != ref.shape:
            raise ValueError(f"{self.label}: shape {got.shape} != reference {ref.shape}")
        self.finite &= bool(np.all(np.isfinite(got)))
        d = got - ref
        self.ss_diff += float(np.sum(d * d))
        self.ss_ref += float(np.sum(ref * ref))
        if d.size:
            self.max_abs = max(self.max_abs, float(np.max(np.abs(d))))
        self.count += got.size

    @property
    def rel(self) -> float:
        return math.sqrt(self.ss_diff) / max(math.sqrt(self.ss_ref), 1e-300)

    @property
    def rms(self) -> float:
        return math.sqrt(self.ss_ref / max(1, self.count))


def compare_all_tokens(outputs: dict, ref_fn, N: int, chunk: int = 1024):
    """outputs: {label: GPU tensor [N, ...]}; ref_fn(lo, hi) -> fp64 numpy reference of tokens lo..hi-1.
    Returns {label: Errors} over every token."""
    errs = {k: Errors(k) for k in outputs}
    for lo in range(0, N, chunk):
        hi = min(N, lo + chunk)
        ref = ref_fn(lo, hi)
        for k, y in outputs.items():
            errs[k].add(y[lo:hi].detach().to("cpu", torch.float64).numpy(), ref)
    return errs
