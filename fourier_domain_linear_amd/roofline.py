"""Algorithmic work and bytes of the EQ-Linear forward, and MI355X peak figures.

Counting follows the Flash EQ-Linear page ("Flash EQ-Linear: Accelerating Equivariant Linear Layers
via Group-wise Discrete Fourier Transform", gist.science/es/paper/2607.21271):

* "Enfoque Algorítmico": after the group DFT, each frequency is an independent channel product, and
  only the non-redundant half k = 0..G/2 of the spectrum is computed. The dense (unrolled) MAC count
  N*D*C (D = C_out*G, C = C_in*G: the unrolled widths) drops to about 2*N*D*C/G.
* "Especialización para el Grupo de Rotación p4": for G = 4 the per-frequency work is six real
  matrix products instead of sixteen (k = 0 and k = 2 are real: one product each; k = 1 is complex:
  four real products).

In general k = 0 and k = G/2 are real (one real product each) and the G/2 - 1 frequencies between
them are complex (four real products each), so the spectral path does 2G - 2 real C_out x C_in
products per token (G = 1: one). Transform adds are O(N*(C_in + C_out)*G) and are not counted.

The dihedral group D4 (order 8; the reflection groups of "Limitaciones y Trabajo Futuro"): four
characters (one real product each) and one 2-D irreducible representation (a 2 x 2 matrix product:
eight real products), twelve per token.
"""
from __future__ import annotations

# MI355X published peaks (dense, no sparsity).
PEAK_HBM_GBS = 8000.0          # HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # fp32 vector / MFMA


def real_products(G: int, group: str = "cyclic") -> int:
    """Real C_out x C_in matrix products per token on the spectral path."""
    if group == "d4":
        if G != 8:
            raise ValueError("D4 has order 8")
        return 12
    if G < 1 or (G & (G - 1)):
        raise ValueError("G must be a power of two")
    return 1 if G == 1 else 2 * G - 2


def spectral_flops(N: int, C_in: int, C_out: int, G: int, group: str = "cyclic") -> int:
    return 2 * N * C_in * C_out * real_products(G, group)


def dense_flops(N: int, C_in: int, C_out: int, G: int) -> int:
    return 2 * N * (C_in * G) * (C_out * G)


def spectral_bytes(N: int, C_in: int, C_out: int, G: int, elem: int) -> int:
    """Bytes the spectral path must move: x, y, the G real weight planes and the bias."""
    return elem * (N * C_in * G + N * C_out * G + C_out * C_in * G + C_out)


def dense_bytes(N: int, C_in: int, C_out: int, G: int, elem: int) -> int:
    """Bytes the unrolled dense product must move: x, y, the (C_out*G) x (C_in*G) weight, the bias."""
    return elem * (N * C_in * G + N * C_out * G + (C_out * G) * (C_in * G) + C_out * G)


def roof_time_s(flops: float, nbytes: float, peak_tflops: float, peak_gbs: float = PEAK_HBM_GBS):
    """(time at the binding roof, 'mfma' or 'hbm')."""
    t_c = flops / (peak_tflops * 1e12)
    t_m = nbytes / (peak_gbs * 1e9)
    return (t_c, "mfma") if t_c >= t_m else (t_m, "hbm")
