"""fp64 oracle for the EQ-Linear layer over the dihedral group D4 (p4m's point group: the four 90-degree
rotations and the four reflections of the square), in plain numpy.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

Source: the Flash EQ-Linear page ("Limitaciones y Trabajo Futuro": generalising the method from the
rotation group p4 to reflection groups) and the EQ-VMamba page (section 5.2: adding reflection
symmetry). The pages give no formulas for it; the layer here is the plainest reading, the group
convolution that the cyclic layer is a special case of ("Percepción Central": weights shared by
shifting along the group):

    y[n, o, h] = b[o] + sum_{i, g} W[o, i, g^-1 h] * x[n, i, g]

with g^-1 h the group's own product. For the cyclic group this is W[o, i, (h - g) mod G].

Elements. Index e = a + 4 b stands for r^a s^b (a = 0..3 rotations by 90 a degrees, b = 1: followed by
the reflection s). The product follows from s r = r^-1 s: r^a s^b . r^c s^d = r^(a + (-1)^b c) s^(b + d).

Fourier transform (the non-abelian analogue of the group DFT, "Enfoque Algorítmico"): for each
irreducible representation rho, F(rho) = sum_g f(g) rho(g). D4 has four 1-D ones (characters
1, (-1)^b, (-1)^a, (-1)^(a+b)) and one 2-D one, the symmetry's own action on the plane: rho(r) the
90-degree rotation [[0, -1], [1, 0]], rho(s) the reflection diag(1, -1). With this convention the
layer becomes, per irrep and channel pair, Y(rho) = X(rho) W(rho) (a 2 x 2 matrix product for the
2-D irrep), and f(g) = (1/8) [sum_chi chi(g) F(chi) + 2 tr(rho(g)^T F(rho))].
"""
from __future__ import annotations

import numpy as np

ORDER = 8


def _f64(a) -> np.ndarray:
    """numpy array or CPU torch tensor (bf16 included) -> float64 numpy array."""
    if hasattr(a, "detach"):
        import torch

        a = a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def element(e: int):
    """(a, b) of element index e = a + 4 b (r^a s^b)."""
    return e % 4, e // 4


def index(a: int, b: int) -> int:
    return (a % 4) + 4 * (b % 2)


def mul(g: int, h: int) -> int:
    """Index of the product g h (r^a s^b r^c s^d = r^(a + (-1)^b c) s^(b + d))."""
    a, b = element(g)
    c, d = element(h)
    return index(a + (c if b == 0 else -c), b + d)


def inv(g: int) -> int:
    """Index of g^-1: rotations invert, reflections are their own inverse."""
    a, b = element(g)
    return index(-a, 0) if b == 0 else g


def expand(W) -> np.ndarray:
    """The unrolled weight E[o*8 + h, i*8 + g] = W[o, i, g^-1 h] (fp64)."""
    W = _f64(W)
    C_out, C_in, G = W.shape
    if G != ORDER:
        raise ValueError(f"D4 weights need a group axis of 8, got {G}")
    idx = np.array([[mul(inv(g), h) for g in range(ORDER)] for h in range(ORDER)])  # [h, g]
    E = W[:, :, idx]                                  # [o, i, h, g]
    return E.transpose(0, 2, 1, 3).reshape(C_out * ORDER, C_in * ORDER)


def forward(x, W, b=None) -> np.ndarray:
    """y[n, o, h] = b[o] + sum_{i, g} W[o, i, g^-1 h] x[n, i, g] in fp64, as the dense product with
    the unrolled weight (numpy's matmul)."""
    x = _f64(x)
    W = _f64(W)
    C_out, C_in, G = W.shape
    if x.ndim != 3 or x.shape[1:] != (C_in, G):
        raise ValueError(f"x shape {x.shape} does not match W shape {W.shape}")
    N = x.shape[0]
    y = x.reshape(N, C_in * G) @ expand(W).T
    if b is not None:
        y = y + np.repeat(_f64(b), G)[None, :]
    return y.reshape(N, C_out, G)


_R = np.array([[0, -1], [1, 0]], dtype=np.float64)
_S = np.array([[1, 0], [0, -1]], dtype=np.float64)


def rho(g: int) -> np.ndarray:
    """The 2-D irrep: rho(r^a s^b) = R^a S^b."""
    a, b = element(g)
    return np.linalg.matrix_power(_R, a) @ np.linalg.matrix_power(_S, b)


def chi(k: int, g: int) -> float:
    """The 1-D irreps k = 0..3: 1, (-1)^b, (-1)^a, (-1)^(a+b)."""
    a, b = element(g)
    return float((1, (-1) ** b, (-1) ** a, (-1) ** (a + b))[k])


def fourier(f) -> np.ndarray:
    """Fourier transform along the last axis (length 8): [..., 8] with the four characters' values
    first, then the 2-D irrep's F(rho) entries (0,0), (0,1), (1,0), (1,1)."""
    f = _f64(f)
    T = np.zeros((8, ORDER))
    for g in range(ORDER):
        for k in range(4):
            T[k, g] = chi(k, g)
        T[4:, g] = rho(g).reshape(4)
    return f @ T.T


def backward_data(dy, W) -> np.ndarray:
    """dx[n, i, g] = sum_{o, h} W[o, i, g^-1 h] dy[n, o, h]: the transpose of the unrolled product."""
    dy = _f64(dy)
    W = _f64(W)
    C_out, C_in, G = W.shape
    N = dy.shape[0]
    return (dy.reshape(N, C_out * G) @ expand(W)).reshape(N, C_in, G)


def backward_weights(x, dy):
    """(dW, db): dE = sum over tokens of dy x^T, folded back onto W (dW[o, i, d] is the sum of dE over
    the (h, g) with g^-1 h = d), db[o] = sum_{n, h} dy[n, o, h]; fp64."""
    x = _f64(x)
    dy = _f64(dy)
    N, C_in, G = x.shape
    C_out = dy.shape[1]
    dE = (dy.reshape(N, C_out * G).T @ x.reshape(N, C_in * G)).reshape(C_out, G, C_in, G)  # [o, h, i, g]
    dW = np.zeros((C_out, C_in, G))
    for h in range(G):
        for g in range(G):
            dW[:, :, mul(inv(g), h)] += dE[:, h, :, g]
    return dW, dy.sum(axis=(0, 2))
