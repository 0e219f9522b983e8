"""fp64 oracle for the p4 group convolution with k x k spatial kernels on the square pixel grid, in
plain numpy.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

Source: the Flash EQ-Linear page ("Limitaciones y Trabajo Futuro": carrying the principle over to
other equivariant operators, equivariant convolutions named among them). The pages give no formula
for it; the layer here is the plainest reading, the rotation-group convolution that the EQ-Linear
layer is the 1 x 1 case of ("Percepción Central": one parameter set shared by cyclic shifts along the
group axis), with the spatial filter turned along with the output orientation:

    y[b, p, o, h] = bias[o] + sum_{i, g} sum_{delta} psi[o, i, (h - g) mod 4, R^-h delta] * x[b, p + delta, i, g]

* p = (row, column) of the pixel, delta = (dy, dx) with |dy|, |dx| <= r = k // 2 (k odd);
* R the 90-degree rotation of an offset, R(dy, dx) = (-dx, dy): the turn numpy's rot90 makes on an
  image whose first axis is the row (np.rot90(a)[p] = a[R^-1 p] about the centre);
* pixels p + delta outside the image contribute zero (zero padding);
* psi[o, i, d, ky, kx] is the filter's value at the offset (ky - r, kx - r).

For k = 1 this is the EQ-Linear layer y[n, o, h] = b[o] + sum W[o, i, (h - g) mod 4] x[n, i, g] with
W = psi[..., 0, 0], one token per pixel. Rotating the image by R (np.rot90 over the two pixel axes)
and shifting the group axis by one commutes with the layer (the grid, the square filter support and
the zero padding are all invariant under R).

Layouts: x[B, H, W, C_in, 4], y[B, H, W, C_out, 4] (one token per pixel, group index innermost, the
layer's own [N, C, G] rows with N = B*H*W), psi[C_out, C_in, 4, k, k], bias[C_out] or None.
"""
from __future__ import annotations

import numpy as np

G = 4


def _f64(a) -> np.ndarray:
    """numpy array or CPU torch tensor (bf16 included) -> float64 numpy array."""
    if hasattr(a, "detach"):
        import torch

        a = a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def rotate_offset(dy: int, dx: int, m: int):
    """R^m (dy, dx) with R(dy, dx) = (-dx, dy); m taken mod 4 (negative m: the inverse turns)."""
    for _ in range(m % 4):
        dy, dx = -dx, dy
    return dy, dx


def shifted(x: np.ndarray, dy: int, dx: int) -> np.ndarray:
    """s[b, py, px] = x[b, py + dy, px + dx] where that pixel lies in the image, else 0."""
    B, H, W = x.shape[:3]
    s = np.zeros_like(x)
    y0, y1 = max(0, -dy), min(H, H - dy)
    x0, x1 = max(0, -dx), min(W, W - dx)
    if y0 < y1 and x0 < x1:
        s[:, y0:y1, x0:x1] = x[:, y0 + dy:y1 + dy, x0 + dx:x1 + dx]
    return s


def forward(x, psi, bias=None) -> np.ndarray:
    """The definition above, summed term by term in fp64 (a matrix product over the input channels as
    the only library step)."""
    x = _f64(x)
    psi = _f64(psi)
    C_out, C_in, g_, k, k2 = psi.shape
    if g_ != G or k != k2 or k % 2 != 1:
        raise ValueError(f"psi must be [C_out, C_in, 4, k, k] with k odd, got {psi.shape}")
    if x.ndim != 5 or x.shape[3:] != (C_in, G):
        raise ValueError(f"x must be [B, H, W, {C_in}, 4], got {x.shape}")
    r = k // 2
    B, H, W = x.shape[:3]
    y = np.zeros((B, H, W, C_out, G), dtype=np.float64)
    for ky in range(k):
        for kx in range(k):
            dy, dx = ky - r, kx - r
            xs = shifted(x, dy, dx)  # x[b, p + delta, i, g]
            for h in range(G):
                fy, fx = rotate_offset(dy, dx, -h)  # R^-h delta: where the filter is read
                for g in range(G):
                    w = psi[:, :, (h - g) % G, fy + r, fx + r]  # [C_out, C_in]
                    y[..., h] += xs[..., g] @ w.T
    if bias is not None:
        y += _f64(bias)[None, None, None, :, None]
    return y
