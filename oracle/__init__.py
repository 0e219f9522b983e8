"""fp64 CPU oracle for the cyclic-group equivariant linear layer (EQ-Linear).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg are the only callers. The GPU library never imports, links or runs anything here,
and nothing here imports the GPU library.

Source followed: "Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise Discrete
Fourier Transform" (explainer page, gist.science/es/paper/2607.21271):

* ``forward`` -- sections "Declaración del Problema" and "Percepción Central": the layer is the
  dense product with the unrolled group-circulant weight E[o*G+h, i*G+g] = W[o, i, (h-g) mod G],
  plus a bias b[o] broadcast over the output group index h. Plain fp64 loops in C
  (``eqlin_oracle.c``); the result the fast method must reproduce ("Principales Contribuciones":
  exact up to floating point).
* ``expand`` -- the unrolled matrix E itself (same section).
* ``dft_weights`` -- section "Enfoque Algorítmico": the DFT of W along the group axis, kept for the
  non-redundant half k = 0..G/2 (conjugate symmetry of a real signal's spectrum).
* ``backward_data``, ``backward_weights`` -- the layer's gradients (section "Implementación": the
  operator has forward and backward kernels), by the chain rule through the unrolled product:
  dx = E^T dy; dE = sum over tokens of dy x^T, folded back onto W along the circulant diagonals
  (dW[o, i, d] = sum_h dE[o*G+h, i*G+(h-d) mod G]); db[o] = sum over tokens and h of dy.
* ``gelu``, ``mlp_block`` -- the transformer MLP block the layer is built into ("Resultados
  Experimentales", network level: EQ-ViT / EQ-Swin), as EQ-Linear(C -> 4C), GELU, EQ-Linear(4C -> C).
  The activation is the GELU the ViT-on-mobile page names ("El Efecto GELU"), in its exact form
  x * Phi(x), Phi the standard normal CDF written with the error function (scipy's erf). Acting on
  each value alone, it commutes with the cyclic shift of the group axis, so the block stays
  equivariant.
* ``dihedral`` (submodule) -- the same layer over the dihedral group D4 (reflections added to the
  p4 rotations), the generalisation the pages name as future work; see its docstring.

All are pinned in ``tests/test_oracle.py`` against things other than themselves (an independent
Kronecker construction of the block-circulant matrix, numpy's FFT convolution theorem, closed forms
for delta / constant / alternating inputs, equivariance, the G=1 plain linear layer; for the
gradients: the adjoint identities <dy, y(x)> = <dx, x> and <dy, y(W)> = <dW, W> against the forward,
central finite differences of a scalar loss, and the G=1 case where dW is the plain dy^T x; for the
block: the normal CDF's table values and its quadrature, GELU(x) - GELU(-x) = x, the G=1 plain MLP,
equivariance, and the saturated cases where GELU is the identity or zero).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import dihedral  # noqa: F401  (oracle.dihedral)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "eqlin_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "libeqlin_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (generic x86-64, -O2, OpenMP). Returns the library path."""
    if not force and os.path.exists(_LIB):
        return _LIB
    os.makedirs(_LIB_DIR, exist_ok=True)
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # EQLIN_ORACLE_LIB: a deliberately broken build of eqlin_oracle.c, used only by the test that
    # checks that the pins catch planted mistakes
    path = os.environ.get("EQLIN_ORACLE_LIB") or _LIB
    if path == _LIB and not os.path.exists(_LIB):
        build(force=False)
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.eqlin_oracle_forward.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, ctypes.c_int]
    lib.eqlin_oracle_forward.restype = ctypes.c_int
    lib.eqlin_oracle_expand.argtypes = [dp, i64, i64, i64, dp]
    lib.eqlin_oracle_expand.restype = ctypes.c_int
    lib.eqlin_oracle_dft_weights.argtypes = [dp, i64, i64, i64, dp, dp]
    lib.eqlin_oracle_dft_weights.restype = ctypes.c_int
    lib.eqlin_oracle_backward_data.argtypes = [dp, dp, dp, i64, i64, i64, i64, ctypes.c_int]
    lib.eqlin_oracle_backward_data.restype = ctypes.c_int
    lib.eqlin_oracle_backward_weights.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, ctypes.c_int]
    lib.eqlin_oracle_backward_weights.restype = ctypes.c_int
    lib.eqlin_oracle_max_threads.argtypes = []
    lib.eqlin_oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    """Any array-like (numpy or a CPU torch tensor) -> C-contiguous float64 numpy array."""
    if hasattr(a, "detach"):  # torch tensor: widen exactly on the torch side (bf16 has no numpy dtype)
        import torch

        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().eqlin_oracle_max_threads())


def forward(x, W, b=None, threads: int = 0) -> np.ndarray:
    """y[n, o, h] = b[o] + sum_{i, g} W[o, i, (h-g) mod G] * x[n, i, g], in fp64.

    x: [N, C_in, G]; W: [C_out, C_in, G]; b: [C_out] or None. ``threads`` = 0 uses OpenMP's default.
    """
    lib = _load()
    W = _f64(W)
    x = _f64(x)
    C_out, C_in, G = W.shape
    if x.ndim != 3 or x.shape[1:] != (C_in, G):
        raise ValueError(f"x shape {x.shape} does not match W shape {W.shape}")
    N = x.shape[0]
    y = np.empty((N, C_out, G), dtype=np.float64)
    bp = None
    if b is not None:
        b = _f64(b)
        if b.shape != (C_out,):
            raise ValueError(f"b shape {b.shape} != ({C_out},)")
        bp = _ptr(b)
    rc = lib.eqlin_oracle_forward(_ptr(x) if N else None, _ptr(W), bp, _ptr(y) if N else None,
                                  N, C_out, C_in, G, int(threads))
    if rc != 0:
        raise RuntimeError(f"eqlin_oracle_forward failed with code {rc}")
    return y


def expand(W) -> np.ndarray:
    """The unrolled block-circulant matrix E[(o*G+h), (i*G+g)] = W[o, i, (h-g) mod G] (fp64)."""
    lib = _load()
    W = _f64(W)
    C_out, C_in, G = W.shape
    E = np.empty((C_out * G, C_in * G), dtype=np.float64)
    rc = lib.eqlin_oracle_expand(_ptr(W), C_out, C_in, G, _ptr(E))
    if rc != 0:
        raise RuntimeError(f"eqlin_oracle_expand failed with code {rc}")
    return E


def dft_weights(W) -> np.ndarray:
    """What[o, i, k] = sum_d W[o, i, d] exp(-2 pi i d k / G) for k = 0..G/2 (complex128)."""
    lib = _load()
    W = _f64(W)
    C_out, C_in, G = W.shape
    K = G // 2 + 1
    re = np.empty((C_out, C_in, K), dtype=np.float64)
    im = np.empty((C_out, C_in, K), dtype=np.float64)
    rc = lib.eqlin_oracle_dft_weights(_ptr(W), C_out, C_in, G, _ptr(re), _ptr(im))
    if rc != 0:
        raise RuntimeError(f"eqlin_oracle_dft_weights failed with code {rc}")
    return re + 1j * im


def backward_data(dy, W, threads: int = 0) -> np.ndarray:
    """dx[n, i, g] = sum_{o, h} W[o, i, (h-g) mod G] * dy[n, o, h] (the transpose of the unrolled
    product), in fp64. dy: [N, C_out, G]; W: [C_out, C_in, G]."""
    lib = _load()
    W = _f64(W)
    dy = _f64(dy)
    C_out, C_in, G = W.shape
    if dy.ndim != 3 or dy.shape[1:] != (C_out, G):
        raise ValueError(f"dy shape {dy.shape} does not match W shape {W.shape}")
    N = dy.shape[0]
    dx = np.empty((N, C_in, G), dtype=np.float64)
    rc = lib.eqlin_oracle_backward_data(_ptr(dy) if N else None, _ptr(W), _ptr(dx) if N else None,
                                        N, C_out, C_in, G, int(threads))
    if rc != 0:
        raise RuntimeError(f"eqlin_oracle_backward_data failed with code {rc}")
    return dx


def backward_weights(x, dy, threads: int = 0):
    """(dW, db): dW[o, i, d] = sum_n sum_h dy[n, o, h] * x[n, i, (h-d) mod G] (through the unrolled
    matrix: dE = dy^T x folded along the circulant diagonals), db[o] = sum_{n, h} dy[n, o, h]; fp64.
    x: [N, C_in, G]; dy: [N, C_out, G]. dW[o, i, :] depends on x[:, i, :] and dy[:, o, :] only, so a
    channel subset of dW is this function of the matching channel slices."""
    lib = _load()
    x = _f64(x)
    dy = _f64(dy)
    if x.ndim != 3 or dy.ndim != 3 or x.shape[0] != dy.shape[0] or x.shape[2] != dy.shape[2]:
        raise ValueError(f"x shape {x.shape} and dy shape {dy.shape} do not match")
    N, C_in, G = x.shape
    C_out = dy.shape[1]
    dW = np.empty((C_out, C_in, G), dtype=np.float64)
    db = np.empty((C_out,), dtype=np.float64)
    rc = lib.eqlin_oracle_backward_weights(_ptr(x) if N else None, _ptr(dy) if N else None, _ptr(dW),
                                           _ptr(db), N, C_out, C_in, G, int(threads))
    if rc != 0:
        raise RuntimeError(f"eqlin_oracle_backward_weights failed with code {rc}")
    return dW, db


def gelu(v) -> np.ndarray:
    """GELU(v) = v * Phi(v) = v/2 * (1 + erf(v / sqrt(2))), elementwise in fp64 (exact form, not the
    tanh approximation)."""
    from scipy.special import erf

    v = _f64(v)
    return 0.5 * v * (1.0 + erf(v / np.sqrt(2.0)))


def mlp_block(x, W1, b1, W2, b2, threads: int = 0) -> np.ndarray:
    """y = EQ-Linear_2(GELU(EQ-Linear_1(x))): W1 [C_h, C, G], b1 [C_h], W2 [C, C_h, G], b2 [C]
    (either bias may be None); x [N, C, G] -> y [N, C_out2, G], fp64 throughout (the hidden
    activation is not rounded)."""
    hidden = gelu(forward(x, W1, b1, threads))
    return forward(hidden, W2, b2, threads)
