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


def test_mfma_counter_summary(tmp_path):
    # two dispatches of one kernel, each counter split over two hardware instances; another kernel's
    # rows must be ignored
    from fourier_domain_linear_amd import profiling

    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows = []
    for d, t0 in ((1, 1000), (2, 5000)):
        for name, v in (("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 240), ("SQ_INSTS_MFMA", 30), ("SQ_INSTS_VALU", 60),
                        ("GRBM_GUI_ACTIVE", 8 * 1200)):
            for _ in range(2):
                rows.append([d, "k_demo<4>", name, v / 2, t0, t0 + 1000])
    rows.append([3, "other", "SQ_INSTS_MFMA", 1e9, 0, 1])
    d = tmp_path / "run"
    d.mkdir()
    with open(d / "x_counter_collection.csv", "w") as f:
        f.write(",".join(hdr) + "\n")
        for r in rows:
            f.write(",".join(f'"{c}"' if isinstance(c, str) else str(c) for c in r) + "\n")
    out = tmp_path / "s.txt"
    profiling.main(["mfma", str(d), "--kernel", "k_demo", "--workload", "p4_c96_n25088_bf16", "--cmd", "c",
                    "--out", str(out)])
    text = out.read_text()
    assert "dispatches averaged: 2" in text
    assert "SQ_INSTS_MFMA: 30 " in text
    # 1024*240 busy cycles over 1024 SIMDs x 1000 ns x 2.4 GHz -> 0.1; over 1200 GRBM cycles per XCD -> 0.2
    assert "over the kernel duration at 2.4 GHz: 0.1000" in text
    assert "over the GRBM_GUI_ACTIVE window: 0.2000" in text
    assert "(2.00 per MFMA)" in text


def test_kernel_stats_summary_with_bench_line(tmp_path):
    # the kernel-trace summary sorted by total time, with the profiled run's own bench figures appended
    import json

    from fourier_domain_linear_amd import profiling

    d = tmp_path / "run"
    d.mkdir()
    with open(d / "k_kernel_stats.csv", "w") as f:
        f.write('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n')
        f.write('"k_small",10,1000,100.0,10.0,90,110,1\n')
        f.write('"k_big",20,9000,450.0,90.0,400,500,1\n')
    line = {"config": {"workload": "p8_c256x1024_n12544_bf16"}, "ms_per_step": 0.1145, "steps": 200,
            "configs": {"p4_c96_n25088_bf16": {"us_per_step": 10.5, "kernel": "bf16 stream"}}}
    bj = tmp_path / "b.json"
    bj.write_text(json.dumps(line))
    out = tmp_path / "s.txt"
    profiling.main(["stats", str(d), "--cmd", "c", "--bench-json", str(bj), "--out", str(out)])
    lines = out.read_text().splitlines()
    rows = [l for l in lines if l.startswith("k_")]
    assert rows[0].split()[0] == "k_big" and rows[1].split()[0] == "k_small"
    assert rows[0].split()[1:3] == ["20", "0.450"]  # calls, average in microseconds
    assert any("p8_c256x1024_n12544_bf16, 114.500 us per step graph-timed over 200 steps" in l for l in lines)
    assert any("p4_c96_n25088_bf16: 10.500 us per step (bf16 stream)" in l for l in lines)
