"""Seeded synthetic workloads for the EQ-Linear forward.

This module holds no arithmetic of the layer itself: it only names the workload shapes and draws
seeded random inputs. It is the one module that both the GPU path's callers (tests, benchmark) and
the fp64 oracle's callers use, so that both sides see the same values.

Shapes. Token counts are flattened vision feature maps (batch x H x W), the activations an EQ-ViT /
EQ-Swin stage feeds its linear layers (Flash EQ-Linear page, "A Nivel de Red"); the pages measured
real networks on ImageNet, which synthetic Gaussian inputs of the same shapes stand in for here.
The group sizes are p4 (G=4, "Especialización para el Grupo de Rotación p4") and its p8 extension
(G=8, 45-degree rotations, the EQ-VMamba page's section 5.2).

Distributions. x ~ N(0, 1); W ~ N(0, 1/(C_in*G)) and b ~ N(0, 0.01), reading the second argument
as the variance, so W has standard deviation (C_in*G)**-0.5 (outputs then have about unit variance)
and b has standard deviation 0.1. Draw order: x, then W, then b, from one ``torch.Generator`` seeded
with ``seed`` (0 by default), in fp32 on the CPU; bf16 workloads are then rounded to bf16 with
round-to-nearest-even, once, and those rounded values are what both the GPU and the oracle see.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    G: int
    C_in: int
    C_out: int
    N: int
    dtype: str  # "f32", "bf16" or "f16"
    group: str = "cyclic"  # or "d4" (G = 8)

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


# The five workloads. The first is the tiny fp32 case the oracle finishes in well under a second;
# the last, the largest single-GPU one (p8, 256 -> 1024 channels, 64x14x14 tokens: the largest
# spectral products, matrix-core bound), is the benchmark's headline workload.
WORKLOADS = [
    Workload("p4_c16_n64_f32", G=4, C_in=16, C_out=16, N=64, dtype="f32"),
    Workload("p4_c96_n25088_bf16", G=4, C_in=96, C_out=96, N=8 * 56 * 56, dtype="bf16"),
    Workload("p8_c64_n25088_bf16", G=8, C_in=64, C_out=64, N=32 * 28 * 28, dtype="bf16"),
    Workload("p4_c192x768_n12544_bf16", G=4, C_in=192, C_out=768, N=16 * 28 * 28, dtype="bf16"),
    Workload("p8_c256x1024_n12544_bf16", G=8, C_in=256, C_out=1024, N=64 * 14 * 14, dtype="bf16"),
]
BY_NAME = {w.name: w for w in WORKLOADS}
BENCH_WORKLOAD = WORKLOADS[4]


def make_inputs(G: int, C_in: int, C_out: int, N: int, dtype: str = "bf16", seed: int = 0):
    """Return CPU tensors (x[N, C_in, G], W[C_out, C_in, G], b[C_out]) in the workload dtype (the same
    fp32 draws, rounded to nearest even for bf16 / f16)."""
    if dtype not in ("f32", "bf16", "f16"):
        raise ValueError(f"dtype must be 'f32', 'bf16' or 'f16', got {dtype!r}")
    gen = torch.Generator().manual_seed(int(seed))
    x = torch.randn((N, C_in, G), generator=gen, dtype=torch.float32)
    W = torch.randn((C_out, C_in, G), generator=gen, dtype=torch.float32) * (C_in * G) ** -0.5
    b = torch.randn((C_out,), generator=gen, dtype=torch.float32) * 0.1
    if dtype != "f32":
        half = torch.bfloat16 if dtype == "bf16" else torch.float16
        x, W, b = x.to(half), W.to(half), b.to(half)
    return x, W, b


def make_grad(G: int, C_out: int, N: int, dtype: str = "bf16", seed: int = 0):
    """An upstream gradient dy[N, C_out, G] ~ N(0, 1) (CPU tensor in the workload dtype) for the
    backward passes; seeded like make_inputs but from its own stream (seed + 7919)."""
    if dtype not in ("f32", "bf16", "f16"):
        raise ValueError(f"dtype must be 'f32', 'bf16' or 'f16', got {dtype!r}")
    gen = torch.Generator().manual_seed(int(seed) + 7919)
    dy = torch.randn((N, C_out, G), generator=gen, dtype=torch.float32)
    return dy if dtype == "f32" else dy.to(torch.bfloat16 if dtype == "bf16" else torch.float16)


def workload_inputs(w: Workload, seed: int = 0, N: int | None = None):
    """Inputs of workload ``w`` (optionally with a different token count N)."""
    return make_inputs(w.G, w.C_in, w.C_out, w.N if N is None else N, w.dtype, seed)


# The MLP block of a transformer stage (EQ-Linear(C -> 4C), GELU, EQ-Linear(4C -> C); the networks of
# "A Nivel de Red") at the p4 MLP-expansion shape: its first layer is the p4_c192x768 workload.
BLOCK_WORKLOAD = Workload("p4_mlp_c192x768x192_n12544_bf16", G=4, C_in=192, C_out=768, N=16 * 28 * 28,
                          dtype="bf16")


def make_block_inputs(G: int, C: int, C_h: int, N: int, dtype: str = "bf16", seed: int = 0):
    """CPU tensors (x[N, C, G], W1[C_h, C, G], b1[C_h], W2[C, C_h, G], b2[C]) for the MLP block:
    x, W1, b1 are make_inputs(G, C, C_h, N, dtype, seed); W2, b2 come from
    make_inputs(G, C_h, C, 0, dtype, seed + 104729) (so W2 ~ N(0, 1/(C_h*G)), b2 ~ N(0, 0.01))."""
    x, W1, b1 = make_inputs(G, C, C_h, N, dtype, seed)
    _, W2, b2 = make_inputs(G, C_h, C, 0, dtype, seed + 104729)
    return x, W1, b1, W2, b2


# The dihedral group D4 (rotations and reflections of the square, order 8) at the two p8 shapes: the
# same tensor sizes as the p8 workloads, a different group.
D4_WORKLOADS = [
    Workload("d4_c64_n25088_bf16", G=8, C_in=64, C_out=64, N=32 * 28 * 28, dtype="bf16", group="d4"),
    Workload("d4_c256x1024_n12544_bf16", G=8, C_in=256, C_out=1024, N=64 * 14 * 14, dtype="bf16", group="d4"),
]
BY_NAME.update({w.name: w for w in D4_WORKLOADS})


# IEEE half precision (the pages' FP16 kernels) at the four half-precision workload shapes.
F16_WORKLOADS = [Workload(w.name.replace("_bf16", "_f16"), G=w.G, C_in=w.C_in, C_out=w.C_out, N=w.N, dtype="f16")
                 for w in WORKLOADS[1:]]
BY_NAME.update({w.name: w for w in F16_WORKLOADS})


# The p4 group convolution with k x k kernels (the equivariant convolutions of "Limitaciones y Trabajo
# Futuro"): one token per pixel of a [B, H, W] batch, x[B, H, W, C_in, 4], psi[C_out, C_in, 4, k, k].
@dataclass(frozen=True)
class ConvWorkload:
    name: str
    C_in: int
    C_out: int
    k: int
    B: int
    H: int
    W: int
    dtype: str = "bf16"

    @property
    def N(self) -> int:
        return self.B * self.H * self.W

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.dtype]


# a 3 x 3 convolution of a vision stage: 256 channels per orientation (1024 with the group axis) on
# 4 feature maps of 64 x 64 pixels
CONV_WORKLOAD = ConvWorkload("p4_conv3x3_c256_n4x64x64_bf16", C_in=256, C_out=256, k=3, B=4, H=64, W=64)


def make_conv_inputs(C_in: int, C_out: int, k: int, B: int, H: int, W: int, dtype: str = "bf16", seed: int = 0):
    """CPU tensors (x[B, H, W, C_in, 4], psi[C_out, C_in, 4, k, k], b[C_out]): x ~ N(0, 1),
    psi ~ N(0, 1/(C_in*4*k*k)) (the layer's reading of the variance: outputs of about unit variance over
    the C_in * 4 * k * k terms), b ~ N(0, 0.01); drawn in that order from one generator, fp32, then rounded
    to nearest even for bf16 / f16."""
    if dtype not in ("f32", "bf16", "f16"):
        raise ValueError(f"dtype must be 'f32', 'bf16' or 'f16', got {dtype!r}")
    gen = torch.Generator().manual_seed(int(seed))
    x = torch.randn((B, H, W, C_in, 4), generator=gen, dtype=torch.float32)
    psi = torch.randn((C_out, C_in, 4, k, k), generator=gen, dtype=torch.float32) * (C_in * 4 * k * k) ** -0.5
    b = torch.randn((C_out,), generator=gen, dtype=torch.float32) * 0.1
    if dtype != "f32":
        half = torch.bfloat16 if dtype == "bf16" else torch.float16
        x, psi, b = x.to(half), psi.to(half), b.to(half)
    return x, psi, b
