"""Pins for the D4 (rotations + reflections) oracle, CPU only. Each checks ``oracle.dihedral``
against something other than itself: the geometric action of the square's symmetries (cos/sin
rotation matrices and a mirror), the group axioms, the pinned cyclic oracle on the rotation
subgroup, brute-force loops, and the representation theory the fast path relies on (Schur
orthogonality and the convolution theorem with the product order X W)."""
import itertools

import numpy as np
import pytest

import oracle
from oracle import dihedral as d4

E8 = range(8)


def _geom(e):
    """The symmetry r^a s^b of the plane, built from angles: rotation by 90a degrees after the mirror
    across the x axis when b = 1."""
    a, b = e % 4, e // 4
    th = a * np.pi / 2
    rot = np.array([[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]])
    mir = np.diag([1.0, -1.0]) if b else np.eye(2)
    return np.round(rot @ mir, 12)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_product_is_the_geometric_composition():
    mats = [_geom(e) for e in E8]
    assert len({m.tobytes() for m in mats}) == 8  # eight distinct symmetries
    for g, h in itertools.product(E8, E8):
        np.testing.assert_array_equal(_geom(d4.mul(g, h)), mats[g] @ mats[h])
    for g in E8:
        np.testing.assert_array_equal(_geom(d4.inv(g)), np.round(np.linalg.inv(mats[g]), 12))


def test_group_axioms_and_non_commutativity():
    for g in E8:
        assert d4.mul(0, g) == g == d4.mul(g, 0)
        assert d4.mul(g, d4.inv(g)) == 0
    for g, h, k in itertools.product(E8, E8, E8):
        assert d4.mul(d4.mul(g, h), k) == d4.mul(g, d4.mul(h, k))
    r, s = 1, 4
    assert d4.mul(r, s) != d4.mul(s, r) and d4.mul(s, r) == d4.mul(d4.inv(r), s)


def test_irreps_are_homomorphisms_and_orthogonal():
    for g, h in itertools.product(E8, E8):
        np.testing.assert_array_equal(d4.rho(d4.mul(g, h)), d4.rho(g) @ d4.rho(h))
        for k in range(4):
            assert d4.chi(k, d4.mul(g, h)) == d4.chi(k, g) * d4.chi(k, h)
    # the 2-D irrep is the geometric action itself
    for g in E8:
        np.testing.assert_array_equal(d4.rho(g), _geom(g))
    # Fourier inversion f(g) = (1/8)[sum_k chi_k(g) F_k + 2 tr(rho(g)^T F_rho)] (Schur orthogonality)
    f = _rand((5, 8), 1)
    F = d4.fourier(f)
    back = np.zeros_like(f)
    for g in E8:
        back[:, g] = (sum(d4.chi(k, g) * F[:, k] for k in range(4))
                      + 2 * (F[:, 4:].reshape(-1, 2, 2) * d4.rho(g)).sum(axis=(1, 2))) / 8
    np.testing.assert_allclose(back, f, rtol=0, atol=1e-13)


def _brute(x, W, b):
    N, C_in, _ = x.shape
    C_out = W.shape[0]
    y = np.zeros((N, C_out, 8))
    for n, o, h in itertools.product(range(N), range(C_out), E8):
        acc = b[o]
        for i, g in itertools.product(range(C_in), E8):
            acc += W[o, i, d4.mul(d4.inv(g), h)] * x[n, i, g]
        y[n, o, h] = acc
    return y


@pytest.mark.parametrize("N,C_out,C_in", [(1, 1, 1), (3, 2, 3)])
def test_forward_matches_brute_force_loops(N, C_out, C_in):
    x, W, b = _rand((N, C_in, 8), 2), _rand((C_out, C_in, 8), 3), _rand((C_out,), 4)
    np.testing.assert_allclose(d4.forward(x, W, b), _brute(x, W, b), rtol=0, atol=1e-12)


def test_equivariance_under_every_symmetry():
    # (t . x)(g) = x(t^-1 g) on the group axis; then y(t . x) = t . y(x) for all eight t
    x, W, b = _rand((4, 3, 8), 5), _rand((5, 3, 8), 6), _rand((5,), 7)
    y = d4.forward(x, W, b)
    for t in E8:
        perm = [d4.mul(d4.inv(t), g) for g in E8]
        np.testing.assert_allclose(d4.forward(x[:, :, perm], W, b), y[:, :, perm], rtol=0, atol=1e-12)


def test_rotation_subgroup_is_the_p4_layer():
    # weights and inputs on the rotations only: the rotation outputs are the cyclic p4 layer (the
    # pinned C oracle), the reflection outputs are the bias alone
    x, W, b = _rand((6, 4, 8), 8), _rand((3, 4, 8), 9), _rand((3,), 10)
    x[:, :, 4:] = 0
    W[:, :, 4:] = 0
    y = d4.forward(x, W, b)
    np.testing.assert_allclose(y[:, :, :4], oracle.forward(x[:, :, :4], W[:, :, :4], b), rtol=0, atol=1e-12)
    np.testing.assert_allclose(y[:, :, 4:], np.broadcast_to(b[None, :, None], (6, 3, 4)), rtol=0, atol=1e-12)


def test_convolution_theorem_product_order():
    # per irrep: Y(chi) = sum_i X_i(chi) W_oi(chi); Y(rho) = sum_i X_i(rho) @ W_oi(rho) -- X on the left
    # (W @ X instead fails: D4 is not commutative)
    x, W = _rand((3, 4, 8), 11), _rand((2, 4, 8), 12)
    Y = d4.fourier(d4.forward(x, W))
    X, Wf = d4.fourier(x), d4.fourier(W)
    for k in range(4):
        np.testing.assert_allclose(Y[:, :, k], X[:, :, k] @ Wf[:, :, k].T, rtol=0, atol=1e-12)
    Xr = X[:, :, 4:].reshape(3, 4, 2, 2)
    Wr = Wf[:, :, 4:].reshape(2, 4, 2, 2)
    ref = np.einsum("niab,oibc->noac", Xr, Wr).reshape(3, 2, 4)
    np.testing.assert_allclose(Y[:, :, 4:], ref, rtol=0, atol=1e-12)
    wrong = np.einsum("oiab,nibc->noac", Wr, Xr).reshape(3, 2, 4)
    assert np.abs(wrong - Y[:, :, 4:]).max() > 1e-3


def test_unrolled_weight_commutes_with_the_group_action():
    W = _rand((2, 3, 8), 13)
    E = d4.expand(W)
    for t in E8:
        P = np.zeros((8, 8))
        for g in E8:
            P[d4.mul(t, g), g] = 1
        np.testing.assert_array_equal(np.kron(np.eye(2), P) @ E, E @ np.kron(np.eye(3), P))


def test_empty_and_bad_shapes():
    assert d4.forward(np.zeros((0, 3, 8)), _rand((2, 3, 8), 14)).shape == (0, 2, 8)
    with pytest.raises(ValueError):
        d4.forward(np.zeros((1, 3, 4)), _rand((2, 3, 4), 15))


def test_backward_adjoint_identities():
    # <dy, y(x)> = <dx, x> (x -> y is linear without bias) and <dy, y(W)> = <dW, W>, against forward
    x, W, dy = _rand((5, 3, 8), 16), _rand((4, 3, 8), 17), _rand((5, 4, 8), 18)
    y = d4.forward(x, W)
    dx = d4.backward_data(dy, W)
    dW, db = d4.backward_weights(x, dy)
    assert abs(np.sum(dy * y) - np.sum(dx * x)) <= 1e-10 * np.abs(dy * y).sum()
    assert abs(np.sum(dy * y) - np.sum(dW * W)) <= 1e-10 * np.abs(dy * y).sum()
    np.testing.assert_allclose(db, dy.sum(axis=(0, 2)), rtol=1e-14)


def test_backward_finite_differences():
    # L = sum(c * y(x, W, b)); central differences along random directions
    x, W, b, c = _rand((3, 2, 8), 19), _rand((3, 2, 8), 20), _rand((3,), 21), _rand((3, 3, 8), 22)
    L = lambda xx, WW, bb: np.sum(c * d4.forward(xx, WW, bb))
    dx = d4.backward_data(c, W)
    dW, db = d4.backward_weights(x, c)
    eps = 1e-6
    for (arg, grad, k) in ((x, dx, 0), (W, dW, 1), (b, db, 2)):
        u = _rand(arg.shape, 23 + k)
        args_p = [x, W, b]
        args_m = [x, W, b]
        args_p[k] = arg + eps * u
        args_m[k] = arg - eps * u
        fd = (L(*args_p) - L(*args_m)) / (2 * eps)
        assert abs(fd - np.sum(grad * u)) <= 1e-6 * max(1.0, abs(fd))
