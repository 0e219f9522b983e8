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


# ---- the gradients (section "Implementación": the operator has forward and backward kernels) ----

# B-1: adjoint identities against the forward. The layer is bilinear in (x, W) plus b, so for any dy
# <dy, y(x, W, 0)> = <dx, x> = <dW, W> and <dy, y(0, 0, b)> = <db, b>. A transposed W, a wrong
# fold direction (h+d instead of h-d) or a dropped group sample breaks one of them.
@pytest.mark.parametrize("G", GROUPS)
def test_backward_adjoint_identities(G):
    N, C_in, C_out = 9, 5, 6
    x, W, b, dy = _rand((N, C_in, G), 40), _rand((C_out, C_in, G), 41), _rand((C_out,), 42), _rand((N, C_out, G), 43)
    lhs = np.sum(dy * oracle.forward(x, W))
    dx = oracle.backward_data(dy, W)
    dW, db = oracle.backward_weights(x, dy)
    assert abs(np.sum(dx * x) - lhs) <= 1e-12 * max(1.0, abs(lhs))
    assert abs(np.sum(dW * W) - lhs) <= 1e-12 * max(1.0, abs(lhs))
    lb = np.sum(dy * oracle.forward(x, np.zeros_like(W), b))
    assert abs(np.sum(db * b) - lb) <= 1e-12 * max(1.0, abs(lb))


# B-2: central finite differences of L = <dy, y(x, W, b)>. L is linear in each argument, so the
# central difference is exact up to rounding; checked entry by entry on a sample.
@pytest.mark.parametrize("G", [2, 4, 8])
def test_backward_finite_differences(G):
    N, C_in, C_out = 4, 3, 5
    x, W, b, dy = _rand((N, C_in, G), 44), _rand((C_out, C_in, G), 45), _rand((C_out,), 46), _rand((N, C_out, G), 47)
    L = lambda x_, W_, b_: float(np.sum(dy * oracle.forward(x_, W_, b_)))
    dx = oracle.backward_data(dy, W)
    dW, db = oracle.backward_weights(x, dy)
    rng = np.random.default_rng(48)
    eps = 0.5
    for _ in range(6):
        n, i, g = rng.integers(N), rng.integers(C_in), rng.integers(G)
        e = np.zeros_like(x)
        e[n, i, g] = eps
        assert abs((L(x + e, W, b) - L(x - e, W, b)) / (2 * eps) - dx[n, i, g]) <= 1e-10
        o, i, d = rng.integers(C_out), rng.integers(C_in), rng.integers(G)
        e = np.zeros_like(W)
        e[o, i, d] = eps
        assert abs((L(x, W + e, b) - L(x, W - e, b)) / (2 * eps) - dW[o, i, d]) <= 1e-10
        o = rng.integers(C_out)
        e = np.zeros_like(b)
        e[o] = eps
        assert abs((L(x, W, b + e) - L(x, W, b - e)) / (2 * eps) - db[o]) <= 1e-10


# B-3: G = 1 is a plain linear layer: dx = dy W, dW = dy^T x, db = column sums of dy.
def test_backward_g1_is_plain_linear():
    x, W, dy = _rand((8, 5, 1), 49), _rand((4, 5, 1), 50), _rand((8, 4, 1), 51)
    np.testing.assert_allclose(oracle.backward_data(dy, W)[:, :, 0], dy[:, :, 0] @ W[:, :, 0], atol=1e-12)
    dW, db = oracle.backward_weights(x, dy)
    np.testing.assert_allclose(dW[:, :, 0], dy[:, :, 0].T @ x[:, :, 0], atol=1e-12)
    np.testing.assert_allclose(db, dy[:, :, 0].sum(axis=0), atol=1e-12)


# B-4: dx through the independently built block-circulant matrix: dx_flat = dy_flat E.
@pytest.mark.parametrize("G", GROUPS)
def test_backward_data_is_transpose_product(G):
    W, dy = _rand((4, 3, G), 52), _rand((6, 4, G), 53)
    ref = (dy.reshape(6, -1) @ _kron_block_circulant(W)).reshape(6, 3, G)
    assert _rel(oracle.backward_data(dy, W), ref) <= 1e-13


# B-5: dW by the correlation theorem with numpy's FFT along the group axis: the DFT of
# c[d] = sum_h dy[h] x[h-d] is DY_k conj(X_k); summed over tokens, then inverted.
@pytest.mark.parametrize("G", GROUPS)
def test_backward_weights_correlation_theorem(G):
    x, dy = _rand((7, 3, G), 54), _rand((7, 5, G), 55)
    C = np.einsum("nok,nik->oik", np.fft.fft(dy, axis=2), np.conj(np.fft.fft(x, axis=2)))
    ref = np.fft.ifft(C, axis=2).real
    dW, db = oracle.backward_weights(x, dy)
    assert _rel(dW, ref) <= 1e-12
    np.testing.assert_allclose(db, dy.sum(axis=(0, 2)), atol=1e-12)


# B-6: a channel subset of dW is the same function of the matching channel slices (the parity tests
# at full token counts rely on this to check sampled channels).
def test_backward_weights_channel_subset():
    x, dy = _rand((6, 7, 4), 56), _rand((6, 5, 4), 57)
    dW, db = oracle.backward_weights(x, dy)
    osub, isub = [0, 3, 4], [1, 2, 6]
    dWs, dbs = oracle.backward_weights(x[:, isub], dy[:, osub])
    np.testing.assert_allclose(dWs, dW[np.ix_(osub, isub)], rtol=0, atol=0)
    np.testing.assert_allclose(dbs, db[osub], rtol=0, atol=0)


def test_backward_empty_batch():
    W = _rand((3, 2, 4), 58)
    assert oracle.backward_data(np.zeros((0, 3, 4)), W).shape == (0, 2, 4)
    dW, db = oracle.backward_weights(np.zeros((0, 2, 4)), np.zeros((0, 3, 4)))
    assert np.all(dW == 0) and np.all(db == 0)


# ---- the MLP block (EQ-Linear(C -> 4C), GELU, EQ-Linear(4C -> C); "Resultados Experimentales",
# network level) and its activation (the ViT-on-mobile page, "El Efecto GELU"). ----

def _phi_quadrature(v):
    """Standard normal CDF by composite Simpson quadrature of the density from 0 to v (independent of
    erf): Phi(v) = 1/2 + int_0^v exp(-t^2/2) / sqrt(2 pi) dt."""
    v = np.asarray(v, dtype=np.float64)
    m = 4000  # even number of panels
    t = np.linspace(0.0, 1.0, m + 1)
    w = np.ones(m + 1)
    w[1:-1:2], w[2:-1:2] = 4.0, 2.0
    pts = v[..., None] * t
    dens = np.exp(-0.5 * pts * pts) / np.sqrt(2.0 * np.pi)
    return 0.5 + v * (dens @ w) / (3.0 * m)


def test_gelu_table_values():
    # Phi(1), Phi(2), Phi(-1) from a standard normal table (15+ digits); GELU(v) = v Phi(v).
    g = oracle.gelu(np.array([0.0, 1.0, -1.0, 2.0]))
    np.testing.assert_allclose(g, [0.0, 0.8413447460685429, -0.15865525393145707, 2 * 0.9772498680518208],
                               rtol=1e-15, atol=0)


def test_gelu_matches_quadrature_cdf():
    v = np.linspace(-6.0, 6.0, 241)
    np.testing.assert_allclose(oracle.gelu(v), v * _phi_quadrature(v), rtol=0, atol=1e-13)


def test_gelu_odd_part_and_limits():
    # Phi(v) + Phi(-v) = 1, so GELU(v) - GELU(-v) = v; GELU -> v for v >> 0 and -> 0 for v << 0.
    v = _rand((1000,), 40) * 3
    np.testing.assert_allclose(oracle.gelu(v) - oracle.gelu(-v), v, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(oracle.gelu(np.array([40.0, -40.0])), [40.0, -0.0])
    # slope 1/2 at 0 (Phi(0) = 1/2)
    assert abs(oracle.gelu(np.array([1e-8]))[0] / 1e-8 - 0.5) < 1e-8


def test_mlp_block_g1_is_plain_mlp():
    # G = 1: x W1^T + b1, GELU (quadrature CDF), then W2^T + b2, all by numpy's matmul.
    N, C, H = 7, 5, 12
    x, W1, b1 = _rand((N, C, 1), 41), _rand((H, C, 1), 42), _rand((H,), 43)
    W2, b2 = _rand((C, H, 1), 44), _rand((C,), 45)
    pre = x[:, :, 0] @ W1[:, :, 0].T + b1
    ref = (pre * _phi_quadrature(pre)) @ W2[:, :, 0].T + b2
    assert _rel(oracle.mlp_block(x, W1, b1, W2, b2)[:, :, 0], ref) <= 1e-12


@pytest.mark.parametrize("G", [2, 4, 8])
def test_mlp_block_equivariance(G):
    x, W1, b1 = _rand((4, 3, G), 46), _rand((12, 3, G), 47), _rand((12,), 48)
    W2, b2 = _rand((3, 12, G), 49), _rand((3,), 50)
    y = oracle.mlp_block(x, W1, b1, W2, b2)
    for s in range(1, G):
        assert _rel(oracle.mlp_block(np.roll(x, s, axis=2), W1, b1, W2, b2), np.roll(y, s, axis=2)) <= 1e-12


@pytest.mark.parametrize("G", [4, 8])
def test_mlp_block_saturated_cases(G):
    # A hidden bias of +60 puts every pre-activation where Phi is 1 in fp64, so the block is the
    # product of the two unrolled matrices (order and biases pinned); -60 zeroes the hidden layer,
    # leaving b2 broadcast over the group axis.
    N, C, H = 5, 3, 12
    x, W1 = _rand((N, C, G), 51) * 0.1, _rand((H, C, G), 52) * 0.1
    W2, b2 = _rand((C, H, G), 53), _rand((C,), 54)
    b1 = np.full(H, 60.0)
    E1, E2 = _kron_block_circulant(W1), _kron_block_circulant(W2)
    hid = x.reshape(N, C * G) @ E1.T + np.repeat(b1, G)
    ref = (hid @ E2.T + np.repeat(b2, G)).reshape(N, C, G)
    assert _rel(oracle.mlp_block(x, W1, b1, W2, b2), ref) <= 1e-13
    y0 = oracle.mlp_block(x, W1, -b1, W2, b2)
    np.testing.assert_allclose(y0, np.broadcast_to(b2[None, :, None], (N, C, G)), rtol=0, atol=1e-12)
