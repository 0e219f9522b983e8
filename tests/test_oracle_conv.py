"""Pins of the p4 group-convolution oracle (oracle/conv.py) against things other than itself.

* k = 1 is the EQ-Linear layer: the pinned C oracle (oracle.forward) on one token per pixel.
* A brute-force evaluation with an explicitly rotated filter bank: for each output orientation h the
  k x k filters psi[o, i, (h - g) mod 4] turned by numpy's rot90 (h quarter turns), then a plain 2-D
  cross-correlation per (o, i, g) with scipy (zero fill) -- no offset arithmetic shared with the oracle.
* Equivariance: turning the image by a quarter (np.rot90 over the pixel axes) and shifting the group
  axis by one gives the same turn and shift of the output (all four turns), while the opposite turn
  does not (the pin tells the two directions apart).
* Translation: a compactly supported input moved inside the image moves the output with it.
* A single nonzero input value reads the filter out: at orientation h = 0 the response around the
  pixel is the point-reflected filter (cross-correlation), printed here as explicit numbers.
* Linearity and the bias.
"""
import numpy as np
import pytest
from scipy.signal import correlate2d

import oracle
from oracle import conv


def _inputs(B, H, W, C_in, C_out, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, H, W, C_in, 4))
    psi = rng.standard_normal((C_out, C_in, 4, k, k))
    b = rng.standard_normal(C_out)
    return x, psi, b


def _turn(y, m):
    """The group action: image turned m quarter turns (np.rot90 over the pixel axes), group axis
    shifted by m."""
    return np.roll(np.rot90(y, m, axes=(1, 2)), m, axis=4)


@pytest.mark.parametrize("C_in,C_out", [(3, 5), (1, 1), (4, 2)])
def test_k1_is_the_eq_linear_layer(C_in, C_out):
    x, psi, b = _inputs(2, 5, 6, C_in, C_out, 1, seed=1)
    got = conv.forward(x, psi, b)
    ref = oracle.forward(x.reshape(-1, C_in, 4), psi[..., 0, 0], b).reshape(got.shape)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("k", [3, 5])
def test_brute_force_rotated_filter_bank(k):
    B, H, W, C_in, C_out = 2, 7, 6, 2, 3
    x, psi, b = _inputs(B, H, W, C_in, C_out, k, seed=2)
    got = conv.forward(x, psi, b)
    ref = np.zeros_like(got)
    for h in range(4):
        for o in range(C_out):
            acc = np.full((B, H, W), b[o])
            for i in range(C_in):
                for g in range(4):
                    filt = np.rot90(psi[o, i, (h - g) % 4], h)  # the filter turned with the orientation
                    for n in range(B):
                        acc[n] += correlate2d(x[n, :, :, i, g], filt, mode="same")
            ref[:, :, :, o, h] = acc
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("k", [3, 5])
@pytest.mark.parametrize("H", [7, 8])
def test_equivariance_under_quarter_turns(k, H):
    x, psi, b = _inputs(2, H, H, 3, 2, k, seed=3)
    y = conv.forward(x, psi, b)
    scale = np.abs(y).max()
    for m in (1, 2, 3):
        err = np.abs(conv.forward(_turn(x, m), psi, b) - _turn(y, m)).max()
        assert err <= 1e-12 * scale, (m, err)
    # the other direction (image turned one way, group shifted the other) is not a symmetry
    wrong = np.roll(np.rot90(x, -1, axes=(1, 2)), 1, axis=4)
    assert np.abs(conv.forward(wrong, psi, b) - np.roll(np.rot90(y, -1, axes=(1, 2)), 1, axis=4)).max() > 1e-3


def test_translation():
    k, H, W = 3, 12, 11
    x, psi, b = _inputs(1, H, W, 2, 3, k, seed=4)
    x[:, :2] = 0
    x[:, -4:] = 0
    x[:, :, :2] = 0
    x[:, :, -4:] = 0  # support well inside the image, room to move by (2, 1)
    y = conv.forward(x, psi, b)
    xs = np.roll(x, (2, 1), axis=(1, 2))
    ys = conv.forward(xs, psi, b)
    np.testing.assert_allclose(ys[:, 3:-1, 2:-1], np.roll(y, (2, 1), axis=(1, 2))[:, 3:-1, 2:-1], atol=1e-12)


def test_single_value_reads_out_the_filter():
    # k = 3, one input channel and one output channel, filter values 1..36 (d-major, then rows, columns)
    psi = np.arange(1.0, 37.0).reshape(1, 1, 4, 3, 3)
    x = np.zeros((1, 5, 5, 1, 4))
    x[0, 2, 2, 0, 1] = 1.0  # pixel (2, 2), group index g0 = 1
    y = conv.forward(x, psi)
    # orientation h = 0 reads d = (0 - 1) mod 4 = 3: psi[0, 0, 3] = [[28, 29, 30], [31, 32, 33], [34, 35, 36]];
    # the output at p = (2, 2) - delta holds psi(delta): the filter reflected through its centre
    expect_h0 = np.array([[36.0, 35.0, 34.0], [33.0, 32.0, 31.0], [30.0, 29.0, 28.0]])
    np.testing.assert_array_equal(y[0, 1:4, 1:4, 0, 0], expect_h0)
    # orientation h = 1 reads d = 0 (values 1..9) at the offset turned back by a quarter:
    # y[(2, 2) - delta] = psi_0(R^-1 delta); e.g. delta = (-1, 0) -> R^-1 delta = (0, 1), psi_0[1, 2] = 6
    assert y[0, 3, 2, 0, 1] == 6.0
    # delta = (0, 1) -> R^-1 delta = (1, 0): psi_0[2, 1] = 8
    assert y[0, 2, 1, 0, 1] == 8.0
    # the centre tap does not turn: h = 2 reads d = 1, centre value 14
    assert y[0, 2, 2, 0, 2] == 14.0
    # outside the 3 x 3 neighbourhood nothing arrives
    assert np.all(y[0, 0, :, 0, :] == 0) and np.all(y[0, :, 4, 0, :] == 0)


def test_linearity_and_bias():
    x, psi, b = _inputs(1, 6, 5, 3, 4, 3, seed=5)
    x2 = np.random.default_rng(6).standard_normal(x.shape)
    y = conv.forward(x, psi)
    np.testing.assert_allclose(conv.forward(2.0 * x - x2, psi), 2.0 * y - conv.forward(x2, psi), atol=1e-12)
    np.testing.assert_array_equal(conv.forward(np.zeros_like(x), psi, b),
                                  np.broadcast_to(b[None, None, None, :, None], y.shape))
    np.testing.assert_allclose(conv.forward(x, psi, b) - y, np.broadcast_to(b[None, None, None, :, None], y.shape),
                               atol=1e-12)
