"""Host-side FLOP/byte accounting against the figures the Flash EQ-Linear page prints
(tests/golden/page_figures.json holds them, each with its section)."""
import json
import os

import pytest

from fourier_domain_linear_amd import roofline

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_p4_six_real_products():
    assert roofline.real_products(4) == GOLD["p4_real_products_flash"]["value"]
    # the naive layer does G*G = 16 real products per (C_out x C_in) block pair
    N, C = 10, 8
    ratio = roofline.dense_flops(N, C, C, 4) / roofline.spectral_flops(N, C, C, 4)
    assert ratio == pytest.approx(GOLD["p4_real_products_naive"]["value"] / 6)
    assert round(ratio, 2) == GOLD["p4_theoretical_speedup"]["value"]


@pytest.mark.parametrize("G", [2, 4, 8, 16, 64])
def test_mac_reduction_about_two_over_T(G):
    # spectral / dense = (2G-2)/G^2, just under 2/G: "N*D*C to about 2*N*D*C/T"
    f = GOLD["mac_reduction_factor_over_T"]["value"]
    r = roofline.spectral_flops(3, 5, 7, G) / roofline.dense_flops(3, 5, 7, G)
    assert r <= f / G
    assert r == pytest.approx(f / G, rel=1.0 / (G - 1) + 1e-12)


def test_g1_is_dense():
    assert roofline.spectral_flops(3, 5, 7, 1) == roofline.dense_flops(3, 5, 7, 1)


def test_bytes_and_roof():
    # p4, 96 channels, 25088 tokens, bf16: x + y = 2 * 25088*96*4*2 bytes, plus weights and bias
    b = roofline.spectral_bytes(25088, 96, 96, 4, 2)
    assert b == 2 * (2 * 25088 * 96 * 4 + 96 * 96 * 4 + 96)
    t, bound = roofline.roof_time_s(roofline.spectral_flops(25088, 96, 96, 4), b, roofline.PEAK_BF16_TFLOPS)
    assert bound == "hbm" and t == pytest.approx(b / 8e12)


def test_bad_group():
    with pytest.raises(ValueError):
        roofline.real_products(3)
