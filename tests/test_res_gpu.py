"""GPU parity of the resident-planes p4 kernel (wide G = 4 layers whose input planes fit on chip)
against the fp64 oracle, through the C ABI.

The kernel keeps one token tile's frequency planes in LDS for every output block, so the cases cover
what its indexing depends on: the tile size (BT = ceil(N / CUs) up to 64, so N below, at and far above
64 per compute unit, and N = 1), the ragged last tile, C_in padded to the weight ring (steps past C_in
read as zeros), the largest C_in whose planes fit (256), C_in = 8 (one step padded to four), output blocks that do
not split evenly over the eight waves and C_out not a multiple of 32 (masked stores), no bias, the GELU epilogue and fp16.
Bars as for the other half-precision paths: bf16 relative Frobenius <= 1e-2 and max abs <= 3e-2;
fp16 the same divided by 8 (three more significant bits in every rounding). These tests prepare with
EQLIN_PREPARE_FIXED_KERNEL, so the resident-planes kernel runs at every N; without it a batch of at most
32 tokens per compute unit runs the large-channel kernel on the same weights (the last test).
"""
import re
import numpy as np
import pytest
import torch

import fourier_domain_linear_amd as eq
import oracle
from fourier_domain_linear_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu

BARS = {"bf16": (1e-2, 3e-2), "f16": (1e-2 / 8, 3e-2 / 8)}


def _check(y_gpu, ref, dtype, label):
    y = y_gpu.detach().to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(y)), label
    diff = y - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    print(f"[parity] {label}: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    r, m = BARS[dtype]
    assert rel <= r and mx <= m, (label, rel, mx)


CASES = [
    (192, 768, 517),     # the p4 MLP expansion's channels, a few tokens per tile
    (192, 768, 1),       # one token
    (200, 280, 3001),    # C_in pads 13 steps to 16; C_out = 8.75 blocks (wave 0 gets two, masked lanes)
    (256, 256, 700),     # the largest C_in: 16 steps (128 KB of planes)
    (192, 256, 40000),   # BT = 64 and 625 tiles (more than the CUs)
    (8, 4096, 300),      # eight input channels (one step padded to four), two tokens per tile
    (96, 1024, 16385),   # BT = 64 with a one-token last tile
]


@pytest.mark.parametrize("with_bias", [True, False], ids=["bias", "nobias"])
@pytest.mark.parametrize("C_in,C_out,N", CASES)
def test_res_forward(C_in, C_out, N, with_bias, cuda_device):
    print(f"[case] res G=4 {C_in}->{C_out} N={N} bias={with_bias}", flush=True)
    x, W, b = make_inputs(4, C_in, C_out, N, "bf16", seed=C_in + C_out + N)
    if not with_bias:
        b = None
    h = eq.prepare_weights(W.to(cuda_device), fixed_kernel=True)
    assert "resident" in h.describe().split("|")[1], h.describe()
    y = eq.forward(h, x.to(cuda_device), None if b is None else b.to(cuda_device))
    torch.cuda.synchronize()
    _check(y, oracle.forward(x, W, b), "bf16", f"res {C_in}->{C_out} N={N} bias={with_bias} [{h.describe()}]")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("C_in,C_out,N", [(192, 768, 517), (200, 280, 3001)])
def test_res_gelu(C_in, C_out, N, dtype, cuda_device):
    print(f"[case] res GELU {dtype} {C_in}->{C_out} N={N}", flush=True)
    x, W, b = make_inputs(4, C_in, C_out, N, dtype, seed=7)
    h = eq.prepare_weights(W.to(cuda_device), fixed_kernel=True)
    y = eq.forward(h, x.to(cuda_device), b.to(cuda_device), act="gelu")
    torch.cuda.synchronize()
    _check(y, oracle.gelu(oracle.forward(x, W, b)), dtype, f"res GELU {dtype} {C_in}->{C_out} N={N}")


@pytest.mark.parametrize("C_in,C_out,N", [(192, 768, 517), (256, 256, 700), (192, 256, 40000)])
def test_res_f16(C_in, C_out, N, cuda_device):
    print(f"[case] res f16 {C_in}->{C_out} N={N}", flush=True)
    x, W, b = make_inputs(4, C_in, C_out, N, "f16", seed=11)
    h = eq.prepare_weights(W.to(cuda_device), fixed_kernel=True)
    assert "resident" in h.describe().split("|")[1], h.describe()
    y = eq.forward(h, x.to(cuda_device), b.to(cuda_device))
    torch.cuda.synchronize()
    assert y.dtype == torch.float16
    _check(y, oracle.forward(x, W, b), "f16", f"res f16 {C_in}->{C_out} N={N}")


def test_res_not_taken_outside_its_range(cuda_device):
    # C_in past the LDS (17 or 20 steps), fewer than eight output blocks: the large-channel kernel instead
    for C_in, C_out in [(264, 512), (320, 256), (192, 224)]:
        x, W, b = make_inputs(4, C_in, C_out, 300, "bf16", seed=5)
        h = eq.prepare_weights(W.to(cuda_device))
        desc = h.describe()
        assert "resident" not in desc.split("|")[1], desc
        y = eq.forward(h, x.to(cuda_device), b.to(cuda_device))
        torch.cuda.synchronize()
        _check(y, oracle.forward(x, W, b), "bf16", f"fallback {C_in}->{C_out} [{desc}]")


def test_batch_size_dispatch(cuda_device):
    # default handle: the large-channel kernel up to the threshold eqlin_describe names, the resident one
    # past it, both on the same spectral weights; a FIXED_KERNEL handle names one kernel only
    C_in, C_out = 192, 768
    x, W, b = make_inputs(4, C_in, C_out, 9000, "bf16", seed=21)
    Wd, bd, xd = W.to(cuda_device), b.to(cuda_device), x.to(cuda_device)
    h = eq.prepare_weights(Wd)
    fwd = h.describe().split("|")[1]
    m = re.search(r"at N <= (\d+): bf16 big", fwd)
    assert m and "resident" in fwd.split(";")[0], fwd
    limit = int(m.group(1))
    assert limit % 32 == 0 and limit >= 32, limit
    hf = eq.prepare_weights(Wd, fixed_kernel=True)
    assert "at N <=" not in hf.describe(), hf.describe()
    for n in sorted({1, 517, min(limit, 9000), min(limit + 1, 9000), 9000}):
        for name, hh in (("default", h), ("fixed", hf)):
            y = eq.forward(hh, xd[:n], bd)
            torch.cuda.synchronize()
            kern = "big" if (hh is h and n <= limit) else "resident"
            _check(y, oracle.forward(x[:n], W, b), "bf16", f"dispatch {name} N={n} ({kern}, limit {limit})")
