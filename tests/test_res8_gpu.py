"""GPU parity of the resident-planes G = 8 kernel (the cyclic group p8 and the dihedral group D4, wide
layers whose input planes fit on chip) against the fp64 oracles, through the C ABI.

The kernel keeps one 32-token tile's eight frequency planes in LDS and hands every workgroup a
contiguous range of (token tile, quad of four 32-output blocks) units, so the cases cover what its
indexing depends on: ranges that start and end inside a tile and cross several tiles (more units than
compute units: N = 40000 at 256 outputs, N = 20000 with one quad per tile), fewer units than compute
units (N = 517, N = 1: a workgroup per unit), the ragged last tile (a one-token tile at N = 4097),
C_in padded to the weight ring (steps past C_in read as zeros; 200 -> 16 steps, 72 -> 8, 8 -> 4), the
largest C_in (256: 128 KB of planes), C_out not a whole number of quads or blocks (280: three quads,
the last with three padded blocks and masked lanes), no bias, the GELU epilogue and fp16.
Bars as for the other half-precision paths: bf16 relative Frobenius <= 1e-2 and max abs <= 3e-2;
fp16 the same divided by 8 (three more significant bits in every rounding).
"""
import numpy as np
import pytest
import torch

import fourier_domain_linear_amd as eq
import oracle
from oracle import dihedral
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


def _ref(x, W, b, group):
    return dihedral.forward(x, W, b) if group == "d4" else oracle.forward(x, W, b)


CASES = [
    (256, 1024, 517),    # the p8 headline's channels, 17 tiles x 8 quads (a workgroup per unit)
    (256, 1024, 1),      # one token
    (200, 280, 3001),    # C_in pads 13 steps to 16; C_out = 8.75 blocks in three quads (masked lanes)
    (256, 256, 40000),   # 1250 tiles x 2 quads over the CUs: ranges start and end inside tiles
    (96, 128, 20000),    # one quad per tile: every unit of a range fills its own tile
    (8, 4096, 300),      # eight input channels (one step padded to four), 32 quads per tile
    (72, 768, 4097),     # C_in pads 5 steps to 8; a one-token last tile
]


@pytest.mark.parametrize("with_bias", [True, False], ids=["bias", "nobias"])
@pytest.mark.parametrize("group", ["cyclic", "d4"])
@pytest.mark.parametrize("C_in,C_out,N", CASES)
def test_res8_forward(C_in, C_out, N, group, with_bias, cuda_device):
    print(f"[case] res8 {group} {C_in}->{C_out} N={N} bias={with_bias}", flush=True)
    x, W, b = make_inputs(8, C_in, C_out, N, "bf16", seed=C_in + C_out + N)
    if not with_bias:
        b = None
    h = eq.prepare_weights(W.to(cuda_device), group=group)
    assert "resident" in h.describe().split("|")[1], h.describe()
    y = eq.forward(h, x.to(cuda_device), None if b is None else b.to(cuda_device))
    torch.cuda.synchronize()
    _check(y, _ref(x, W, b, group), "bf16", f"res8 {group} {C_in}->{C_out} N={N} bias={with_bias} [{h.describe()}]")


@pytest.mark.parametrize("group", ["cyclic", "d4"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("C_in,C_out,N", [(256, 1024, 517), (200, 280, 3001)])
def test_res8_gelu(C_in, C_out, N, dtype, group, cuda_device):
    print(f"[case] res8 GELU {dtype} {group} {C_in}->{C_out} N={N}", flush=True)
    x, W, b = make_inputs(8, C_in, C_out, N, dtype, seed=7)
    h = eq.prepare_weights(W.to(cuda_device), group=group)
    y = eq.forward(h, x.to(cuda_device), b.to(cuda_device), act="gelu")
    torch.cuda.synchronize()
    _check(y, oracle.gelu(_ref(x, W, b, group)), dtype, f"res8 GELU {dtype} {group} {C_in}->{C_out} N={N}")


@pytest.mark.parametrize("group", ["cyclic", "d4"])
@pytest.mark.parametrize("C_in,C_out,N", [(256, 1024, 517), (256, 256, 40000), (72, 768, 4097)])
def test_res8_f16(C_in, C_out, N, group, cuda_device):
    print(f"[case] res8 f16 {group} {C_in}->{C_out} N={N}", flush=True)
    x, W, b = make_inputs(8, C_in, C_out, N, "f16", seed=11)
    h = eq.prepare_weights(W.to(cuda_device), group=group)
    assert "resident" in h.describe().split("|")[1], h.describe()
    y = eq.forward(h, x.to(cuda_device), b.to(cuda_device))
    torch.cuda.synchronize()
    assert y.dtype == torch.float16
    _check(y, _ref(x, W, b, group), "f16", f"res8 f16 {group} {C_in}->{C_out} N={N}")


def test_res8_not_taken_outside_its_range(cuda_device):
    # C_in past the LDS (17 or 20 steps): the large-channel kernel; few channels: the stream kernel
    for C_in, C_out in [(264, 512), (320, 256), (64, 64)]:
        x, W, b = make_inputs(8, C_in, C_out, 300, "bf16", seed=5)
        h = eq.prepare_weights(W.to(cuda_device))
        desc = h.describe()
        assert "resident" not in desc.split("|")[1], desc
        y = eq.forward(h, x.to(cuda_device), b.to(cuda_device))
        torch.cuda.synchronize()
        _check(y, oracle.forward(x, W, b), "bf16", f"fallback {C_in}->{C_out} [{desc}]")
