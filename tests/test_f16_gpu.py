"""GPU parity of the IEEE half-precision path (EQLIN_F16: the FP16 kernels the Flash EQ-Linear page
lists under "Implementación") against the fp64 oracle fed the same fp16-rounded inputs.

Bar, derived from the arithmetic: the fp16 path runs the bf16 path's steps (fp32 transforms, one
rounding of the x and weight planes to the half type, fp32 accumulation, one rounding of y), and fp16
keeps 11 significant bits against bf16's 8, so every rounding error is 8x smaller: the bf16 bars
divided by 8 -- relative Frobenius error <= 1.25e-3 AND max abs error <= 3.75e-3 (gradients: max abs
<= 3.75e-3 * rms(reference)).
"""
import numpy as np
import pytest
import torch

import fourier_domain_linear_amd as eq
import oracle
from fourier_domain_linear_amd.workloads import F16_WORKLOADS, make_grad, make_inputs
from oracle import dihedral as d4
from fullsize import compare_all_tokens

pytestmark = pytest.mark.gpu

REL_F16, MAX_F16 = 1e-2 / 8, 3e-2 / 8


def _check(y_gpu, ref, label, max_scale=1.0):
    y = y_gpu.detach().to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(y)), label
    diff = y - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    print(f"[parity] {label}: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= REL_F16 and mx <= MAX_F16 * max_scale, (label, rel, mx)


CASES = [(4, 96, 96, 517), (8, 64, 64, 517), (2, 64, 72, 300), (1, 64, 40, 300), (4, 40, 20, 130),
         (4, 192, 768, 517), (8, 256, 1024, 300), (4, 128, 4095, 200), (4, 64, 64, 1)]


@pytest.mark.parametrize("expanded", [False, True], ids=["spectral", "expanded"])
@pytest.mark.parametrize("G,C_in,C_out,N", CASES)
def test_forward(G, C_in, C_out, N, expanded, cuda_device):
    print(f"[case] f16 G={G} {C_in}->{C_out} N={N} expanded={expanded}", flush=True)
    x, W, b = make_inputs(G, C_in, C_out, N, "f16", seed=31)
    h = eq.prepare_weights(W.to(cuda_device), expanded=expanded)
    y = (eq.forward_expanded if expanded else eq.forward)(h, x.to(cuda_device), b.to(cuda_device))
    torch.cuda.synchronize()
    assert y.dtype == torch.float16
    _check(y, oracle.forward(x, W, b), f"f16 G={G} {C_in}->{C_out} N={N} {'expanded' if expanded else 'spectral'} "
           f"[{h.describe()}]")


@pytest.mark.parametrize("w", F16_WORKLOADS, ids=[w.name for w in F16_WORKLOADS])
def test_full_size_all_tokens(w, cuda_device):
    x, W, b = make_inputs(w.G, w.C_in, w.C_out, w.N, "f16", seed=0)
    h = eq.prepare_weights(W.to(cuda_device))
    y = eq.forward(h, x.to(cuda_device), b.to(cuda_device))
    torch.cuda.synchronize()
    e = compare_all_tokens({"y": y}, lambda lo, hi: oracle.forward(x[lo:hi], W, b), w.N, chunk=2048)["y"]
    print(f"[parity] {w.name} all {w.N} tokens: rel_frob={e.rel:.3e} max_abs={e.max_abs:.3e}", flush=True)
    assert e.finite and e.rel <= REL_F16 and e.max_abs <= MAX_F16, (w.name, e.rel, e.max_abs)


@pytest.mark.parametrize("C_in,C_out", [(64, 64), (256, 1024)])
def test_d4_and_gelu(C_in, C_out, cuda_device):
    x, W, b = make_inputs(8, C_in, C_out, 300, "f16", seed=32)
    h = eq.prepare_weights(W.to(cuda_device), group="d4")
    y = eq.forward(h, x.to(cuda_device), b.to(cuda_device))
    z = eq.forward(h, x.to(cuda_device), b.to(cuda_device), act="gelu")
    torch.cuda.synchronize()
    ref = d4.forward(x, W, b)
    _check(y, ref, f"f16 d4 {C_in}->{C_out}")
    _check(z, oracle.gelu(ref), f"f16 d4 gelu {C_in}->{C_out}")


def test_spectral_weights_and_backward(cuda_device):
    x, W, _ = make_inputs(4, 64, 96, 400, "f16", seed=33)
    dy = make_grad(4, 96, 400, "f16", seed=33)
    h = eq.prepare_weights(W.to(cuda_device), backward=True)
    Wf = eq.export_spectral_weights(h).cpu().double().numpy()
    Wh = oracle.dft_weights(W)  # [C_out, C_in, 3] complex
    ref = np.stack([Wh[..., 0].real, Wh[..., 2].real, Wh[..., 1].real, Wh[..., 1].imag])
    assert np.max(np.abs(Wf - ref) / np.maximum(np.abs(ref), 1e-3)) <= 2 ** -11 * 1.01  # one fp16 rounding
    dx = eq.backward_data(h, dy.to(cuda_device))
    dW, db = eq.backward_weights(h, x.to(cuda_device), dy.to(cuda_device))
    torch.cuda.synchronize()
    rms = lambda a: float(np.sqrt(np.mean(a * a)))
    ref_dx = oracle.backward_data(dy, W)
    ref_dW, ref_db = oracle.backward_weights(x, dy)
    _check(dx, ref_dx, "f16 dx", rms(ref_dx))
    _check(dW, ref_dW, "f16 dW", rms(ref_dW))
    _check(db, ref_db, "f16 db", rms(ref_db))


@pytest.mark.parametrize("group", ["cyclic", "d4"])
def test_backward_weights_fused_g8(group, cuda_device):
    # fp16 at G = 8 and small channel counts: the fused matrix-core weight gradient
    x, W, _ = make_inputs(8, 64, 64, 3001, "f16", seed=34)
    dy = make_grad(8, 64, 3001, "f16", seed=34)
    h = eq.prepare_weights(W.to(cuda_device), group=group)
    assert "fused" in h.describe()
    dW, db = eq.backward_weights(h, x.to(cuda_device), dy.to(cuda_device))
    torch.cuda.synchronize()
    rW, rb = (d4.backward_weights(x, dy) if group == "d4" else oracle.backward_weights(x, dy))
    rms = lambda a: float(np.sqrt(np.mean(a * a)))
    _check(dW, rW, f"f16 {group} dW fused", rms(rW))
    _check(db, rb, f"f16 {group} db fused", rms(rb))


@pytest.mark.parametrize("G,C_in,C_out,N,group", [(4, 192, 768, 300, "cyclic"), (8, 256, 1024, 130, "cyclic"),
                                                   (8, 256, 1024, 130, "d4")])
def test_backward_weights_large_channels(G, C_in, C_out, N, group, cuda_device):
    # fp16 at large channel counts: the three-pass matrix-core weight gradient
    x, W, _ = make_inputs(G, C_in, C_out, N, "f16", seed=35)
    dy = make_grad(G, C_out, N, "f16", seed=35)
    h = eq.prepare_weights(W.to(cuda_device), group=group)
    assert "split-K" in h.describe()
    dW, db = eq.backward_weights(h, x.to(cuda_device), dy.to(cuda_device))
    torch.cuda.synchronize()
    rW, rb = d4.backward_weights(x, dy) if group == "d4" else oracle.backward_weights(x, dy)
    rms = lambda a: float(np.sqrt(np.mean(a * a)))
    _check(dW, rW, f"f16 dW G={G} {C_in}x{C_out}", rms(rW))
    _check(db, rb, f"f16 db G={G} {C_in}x{C_out}", rms(rb))
