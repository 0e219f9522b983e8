"""The kernels' G-point DFT butterflies (csrc/dft.h, compiled for the host) against numpy's FFT.

Plane order (csrc/dft.h): Re X_0, Re X_{G/2}, then Re/Im of X_1 .. X_{G/2-1}. The inverse takes
products already scaled by 1/G (real planes) and 2/G (complex planes). Flash EQ-Linear page,
"Enfoque Algorítmico" (half spectrum) and "Especialización para el Grupo de Rotación p4".
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    out = tmp_path_factory.mktemp("dft") / "libdftshim.so"
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", os.path.join(HERE, "native", "dft_shim.cpp"),
                    "-o", str(out)], check=True)
    lib = ctypes.CDLL(str(out))
    fp = ctypes.POINTER(ctypes.c_float)
    lib.dft_forward.argtypes = [ctypes.c_int, fp, fp]
    lib.dft_inverse.argtypes = [ctypes.c_int, fp, fp]
    lib.dft_plane_scale.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.dft_plane_scale.restype = ctypes.c_float
    lib.d4_forward.argtypes = [fp, fp]
    lib.d4_inverse.argtypes = [fp, fp]
    lib.d4_plane_scale.argtypes = [ctypes.c_int]
    lib.d4_plane_scale.restype = ctypes.c_float
    return lib


def _call(fn, G, v):
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(G, dtype=np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    assert fn(G, v.ctypes.data_as(fp), out.ctypes.data_as(fp)) == 0
    return out


def _planes_from_rfft(X, G):
    if G == 1:
        return np.array([X[0].real])
    p = [X[0].real, X[G // 2].real]
    for k in range(1, G // 2):
        p += [X[k].real, X[k].imag]
    return np.array(p)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_forward_matches_rfft(shim, G):
    rng = np.random.default_rng(G)
    for _ in range(50):
        v = rng.standard_normal(G).astype(np.float32)
        ref = _planes_from_rfft(np.fft.rfft(v.astype(np.float64)), G)
        np.testing.assert_allclose(_call(shim.dft_forward, G, v), ref, rtol=0, atol=2e-6)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_inverse_matches_irfft(shim, G):
    rng = np.random.default_rng(10 + G)
    scale = np.array([shim.dft_plane_scale(G, p) for p in range(G)])
    for _ in range(50):
        y = rng.standard_normal(G)
        Y = _planes_from_rfft(np.fft.rfft(y), G) * scale
        np.testing.assert_allclose(_call(shim.dft_inverse, G, Y), y, rtol=0, atol=2e-6)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_round_trip_convolution(shim, G):
    # y = irfft(rfft(W) * rfft(x)) through the butterflies: the per-frequency product written out.
    rng = np.random.default_rng(20 + G)
    scale = np.array([shim.dft_plane_scale(G, p) for p in range(G)])
    for _ in range(20):
        x, w = rng.standard_normal(G), rng.standard_normal(G)
        X = _call(shim.dft_forward, G, x).astype(np.float64)
        Wp = _call(shim.dft_forward, G, w).astype(np.float64) * scale
        Y = np.empty(G)
        Y[0] = X[0] * Wp[0]
        if G >= 2:
            Y[1] = X[1] * Wp[1]
        for k in range(1, G // 2):
            r, i = 2 * k, 2 * k + 1
            Y[r] = X[r] * Wp[r] - X[i] * Wp[i]
            Y[i] = X[r] * Wp[i] + X[i] * Wp[r]
        ref = np.array([sum(w[(h - g) % G] * x[g] for g in range(G)) for h in range(G)])
        np.testing.assert_allclose(_call(shim.dft_inverse, G, Y), ref, rtol=0, atol=1e-5)


def test_p4_needs_no_multiplies(shim):
    # "Especialización ... p4": forward coefficients are 0 and +-1 -- the transform of a unit vector
    # is exactly representable (no rounding), i.e. only adds/subtracts are involved.
    for d in range(4):
        e = np.zeros(4, dtype=np.float32)
        e[d] = 1.0
        P = _call(shim.dft_forward, 4, e)
        assert set(np.unique(P)).issubset({-1.0, 0.0, 1.0})
    assert [shim.dft_plane_scale(4, p) for p in range(4)] == [0.25, 0.25, 0.5, 0.5]


# ---- D4 (rotations + reflections): the kernels' butterflies against the oracle's irreps ----

def _d4(fn, v):
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(8, dtype=np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    fn(v.ctypes.data_as(fp), out.ctypes.data_as(fp))
    return out


def test_d4_forward_matches_irreps(shim):
    from oracle import dihedral

    rng = np.random.default_rng(31)
    for _ in range(50):
        v = rng.standard_normal(8).astype(np.float32)
        np.testing.assert_allclose(_d4(shim.d4_forward, v), dihedral.fourier(v.astype(np.float64)),
                                   rtol=0, atol=2e-6)
    # coefficients 0 / +-1 only
    for e in range(8):
        u = np.zeros(8, dtype=np.float32)
        u[e] = 1
        assert set(np.unique(_d4(shim.d4_forward, u))).issubset({-1.0, 0.0, 1.0})


def test_d4_inverse_and_group_convolution(shim):
    # x, w -> planes; Y = X W per irrep (characters: products; rho: 2 x 2 product X @ W) with the
    # scales; inverse -> the group convolution y(h) = sum_g w(g^-1 h) x(g) written with the oracle's
    # group product
    from oracle import dihedral as d4

    rng = np.random.default_rng(32)
    scale = np.array([shim.d4_plane_scale(p) for p in range(8)])
    assert list(scale) == [0.125] * 4 + [0.25] * 4
    for _ in range(30):
        x, w = rng.standard_normal(8), rng.standard_normal(8)
        X = _d4(shim.d4_forward, x).astype(np.float64)
        Wp = _d4(shim.d4_forward, w).astype(np.float64) * scale
        Y = np.empty(8)
        Y[:4] = X[:4] * Wp[:4]
        Y[4:] = (X[4:].reshape(2, 2) @ Wp[4:].reshape(2, 2)).reshape(4)
        ref = np.array([sum(w[d4.mul(d4.inv(g), h)] * x[g] for g in range(8)) for h in range(8)])
        np.testing.assert_allclose(_d4(shim.d4_inverse, Y), ref, rtol=0, atol=2e-5)
