"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself, chosen so that a plausible slip in
the oracle (a dropped bias, a sign flip h+g vs h-g, a transposed W, a wrong spectral sign) fails at
least one of them. Page citations refer to "Flash EQ-Linear: Accelerating Equivariant Linear Layers
via Group-wise Discrete Fourier Transform" (explainer, gist.science/es/paper/2607.21271) unless
stated otherwise.
"""
import itertools

import numpy as np
import pytest

import oracle

GROUPS = [1, 2, 4, 8]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _kron_block_circulant(W):
    """Independent construction of the unrolled weight: sum_d W[:, :, d] (x) P^d, where P is the
    G x G cyclic shift (P^d)[h, g] = 1 iff h = g + d (mod G). Section "Percepción Central": the
    dense weight is formed by cyclically shifting and replicating one parameter set."""
    C_out, C_in, G = W.shape
    E = np.zeros((C_out * G, C_in * G))
    for d in range(G):
        Pd = np.roll(np.eye(G), d, axis=0)
        E += np.kron(W[:, :, d], Pd)
    return E


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# P-1: brute force against an independently built block-circulant matrix on tiny shapes.
@pytest.mark.parametrize("G", GROUPS)
@pytest.mark.parametrize("C_out,C_in", [(1, 1), (2, 3), (3, 2)])
def test_expand_matches_kronecker_construction(G, C_out, C_in):
    W = _rand((C_out, C_in, G), 1)
    E = oracle.expand(W)
    np.testing.assert_array_equal(E, _kron_block_circulant(W))


@pytest.mark.parametrize("G", GROUPS)
def test_expand_is_block_circulant(G):
    # Section "Percepción Central": shifting the output and input group index together leaves E fixed.
    C_out, C_in = 3, 2
    E = oracle.expand(_rand((C_out, C_in, G), 2)).reshape(C_out, G, C_in, G)
    for h, g in itertools.product(range(G), range(G)):
        np.testing.assert_array_equal(E[:, h, :, g], E[:, (h + 1) % G, :, (g + 1) % G])


@pytest.mark.parametrize("G", GROUPS)
@pytest.mark.parametrize("N,C_out,C_in", [(1, 1, 1), (5, 2, 3), (4, 3, 2)])
def test_forward_matches_dense_product(G, N, C_out, C_in):
    x, W, b = _rand((N, C_in, G), 3), _rand((C_out, C_in, G), 4), _rand((C_out,), 5)
    y = oracle.forward(x, W, b)
    E = _kron_block_circulant(W)
    ref = (x.reshape(N, C_in * G) @ E.T + np.repeat(b, G)[None, :]).reshape(N, C_out, G)
    assert _rel(y, ref) <= 1e-13


# P-2: rotation equivariance, cyclic shift of the group axis (sections "Resumen"/"Principales
# Contribuciones": the method keeps the operator's rotation equivariance; EQ-VMamba page §3.1).
@pytest.mark.parametrize("G", [2, 4, 8])
def test_equivariance(G):
    x, W, b = _rand((6, 5, G), 6), _rand((7, 5, G), 7), _rand((7,), 8)
    y = oracle.forward(x, W, b)
    for s in range(1, G):
        ys = oracle.forward(np.roll(x, s, axis=2), W, b)
        assert _rel(ys, np.roll(y, s, axis=2)) <= 1e-12


# P-3: G = 1 is a plain linear layer y = x W^T + b (numpy's matmul).
def test_g1_is_plain_linear():
    x, W, b = _rand((9, 6, 1), 9), _rand((4, 6, 1), 10), _rand((4,), 11)
    y = oracle.forward(x, W, b)
    ref = x[:, :, 0] @ W[:, :, 0].T + b
    assert _rel(y[:, :, 0], ref) <= 1e-13


# P-4: group-constant input: y[n, o, h] = sum_i (sum_d W[o, i, d]) c[n, i] + b[o] for every h.
@pytest.mark.parametrize("G", GROUPS)
def test_group_constant_input(G):
    c = _rand((5, 4), 12)
    W, b = _rand((3, 4, G), 13), _rand((3,), 14)
    x = np.repeat(c[:, :, None], G, axis=2)
    y = oracle.forward(x, W, b)
    ref = c @ W.sum(axis=2).T + b
    for h in range(G):
        assert _rel(y[:, :, h], ref) <= 1e-13


# P-5: a delta at input channel i, group element s: y[o, h] = W[o, i, (h - s) mod G] + b[o], exactly.
@pytest.mark.parametrize("G", GROUPS)
def test_delta_input_reads_out_weights(G):
    C_out, C_in = 3, 4
    W, b = _rand((C_out, C_in, G), 15), _rand((C_out,), 16)
    for i, s in itertools.product(range(C_in), range(G)):
        x = np.zeros((1, C_in, G))
        x[0, i, s] = 1.0
        y = oracle.forward(x, W, b)[0]
        for h in range(G):
            np.testing.assert_array_equal(y[:, h], W[:, i, (h - s) % G] + b)


# P-6: alternating input (-1)^g c pins the k = G/2 frequency:
# y[n, o, h] = (-1)^h sum_i (sum_d (-1)^d W[o, i, d]) c[n, i] + b[o].
@pytest.mark.parametrize("G", [2, 4, 8])
def test_alternating_input(G):
    c = _rand((5, 3), 17)
    W, b = _rand((4, 3, G), 18), _rand((4,), 19)
    sgn = (-1.0) ** np.arange(G)
    x = c[:, :, None] * sgn[None, None, :]
    y = oracle.forward(x, W, b)
    core = c @ (W * sgn[None, None, :]).sum(axis=2).T
    for h in range(G):
        assert _rel(y[:, :, h] - b, sgn[h] * core) <= 1e-13


# P-7: zero input gives the bias; the layer is affine (linear part).
@pytest.mark.parametrize("G", GROUPS)
def test_zero_and_linearity(G):
    W, b = _rand((3, 4, G), 20), _rand((3,), 21)
    y0 = oracle.forward(np.zeros((2, 4, G)), W, b)
    np.testing.assert_array_equal(y0, np.broadcast_to(b[None, :, None], y0.shape))
    x1, x2 = _rand((3, 4, G), 22), _rand((3, 4, G), 23)
    a1, a2 = 0.75, -1.5
    lhs = oracle.forward(a1 * x1 + a2 * x2, W, b) - b[None, :, None]
    rhs = a1 * (oracle.forward(x1, W, b) - b[None, :, None]) + a2 * (oracle.forward(x2, W, b) - b[None, :, None])
    assert _rel(lhs, rhs) <= 1e-13
    yn = oracle.forward(x1, W, None)
    assert _rel(yn, oracle.forward(x1, W, b) - b[None, :, None]) <= 1e-13


# P-8: the convolution theorem with numpy's real FFT along the group axis (section "Enfoque
# Algorítmico"): Y_k = sum_i What[o, i, k] X[n, i, k], y = irfft(Y) + b.
@pytest.mark.parametrize("G", GROUPS)
def test_convolution_theorem_numpy_fft(G):
    x, W, b = _rand((7, 6, G), 24), _rand((5, 6, G), 25), _rand((5,), 26)
    X = np.fft.rfft(x, axis=2)
    Wh = np.fft.rfft(W, axis=2)
    Y = np.einsum("oik,nik->nok", Wh, X)
    ref = np.fft.irfft(Y, n=G, axis=2) + b[None, :, None]
    assert _rel(oracle.forward(x, W, b), ref) <= 1e-12


# The spectral weights: numpy's rfft, and the p4 closed form with dyadic coefficients
# (section "Especialización para el Grupo de Rotación p4").
@pytest.mark.parametrize("G", GROUPS)
def test_dft_weights_match_numpy_rfft(G):
    W = _rand((4, 3, G), 27)
    np.testing.assert_allclose(oracle.dft_weights(W), np.fft.rfft(W, axis=2), rtol=0, atol=1e-14)


def test_dft_weights_p4_closed_form():
    W = _rand((3, 5, 4), 28)
    Wh = oracle.dft_weights(W)
    w0, w1, w2, w3 = (W[:, :, d] for d in range(4))
    np.testing.assert_allclose(Wh[:, :, 0], w0 + w1 + w2 + w3, atol=1e-15)
    np.testing.assert_allclose(Wh[:, :, 2], w0 - w1 + w2 - w3, atol=1e-15)
    np.testing.assert_allclose(Wh[:, :, 1], (w0 - w2) - 1j * (w1 - w3), atol=1e-15)


def test_p4_transform_coefficients_are_dyadic():
    # Section "Especialización para el Grupo de Rotación p4": the p4 DFT matrix holds only 0 and +-1
    # in its real and imaginary parts (the inverse adds +-1/2 and 1/4-type scalings).
    G = 4
    cols = [oracle.dft_weights(np.eye(G)[d].reshape(1, 1, G))[0, 0] for d in range(G)]
    F = np.stack(cols, axis=1)  # F[k, d]
    vals = np.concatenate([F.real.ravel(), F.imag.ravel()])
    assert np.all(np.min(np.abs(vals[:, None] - np.array([-1.0, 0.0, 1.0])[None, :]), axis=1) < 1e-15)


def test_empty_batch():
    W, b = _rand((3, 2, 4), 29), _rand((3,), 30)
    y = oracle.forward(np.zeros((0, 2, 4)), W, b)
    assert y.shape == (0, 3, 4)


def test_bad_shapes_raise():
    with pytest.raises(ValueError):
        oracle.forward(np.zeros((2, 3, 4)), np.zeros((3, 2, 4)))
