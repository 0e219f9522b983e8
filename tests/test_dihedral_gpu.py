"""GPU parity for the EQ-Linear layer over the dihedral group D4 (rotations and reflections of the
square; EQLIN_PREPARE_D4) against ``oracle.dihedral`` (fp64 dense product with the unrolled group
convolution). Reflection groups are the generalisation the Flash EQ-Linear page names as future work
("Limitaciones y Trabajo Futuro").

Bars: the layer's own -- bf16: relative Frobenius error <= 1e-2 AND max abs error <= 3e-2 against the
oracle fed the same bf16-rounded inputs; fp32: relative Frobenius error <= 1e-5. Gradients: the same
relative bar and max-abs <= 3e-2 * rms(reference) (they are not unit-scale), as for the cyclic group.
"""
import numpy as np
import pytest
import torch

import fourier_domain_linear_amd as eq
from fourier_domain_linear_amd.workloads import D4_WORKLOADS, make_grad, make_inputs
from oracle import dihedral as d4
from fullsize import compare_all_tokens

pytestmark = pytest.mark.gpu

REL_BF16, MAX_BF16, REL_F32 = 1e-2, 3e-2, 1e-5


def _check(y_gpu, ref, dtype, label, max_scale=1.0):
    y = y_gpu.detach().to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(y)), label
    diff = y - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    print(f"[parity] {label}: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    if dtype == "bf16":
        assert rel <= REL_BF16 and mx <= MAX_BF16 * max_scale, (label, rel, mx)
    else:
        assert rel <= REL_F32, (label, rel)


CASES = [("bf16", 32, 32, 517), ("bf16", 64, 64, 517), ("bf16", 64, 20, 130), ("bf16", 40, 72, 300),
         ("bf16", 256, 1024, 300), ("bf16", 128, 200, 200), ("bf16", 64, 64, 1), ("bf16", 64, 64, 17),
         ("f32", 16, 16, 64), ("f32", 24, 40, 77)]


@pytest.mark.parametrize("with_bias", [True, False], ids=["bias", "nobias"])
@pytest.mark.parametrize("expanded", [False, True], ids=["spectral", "expanded"])
@pytest.mark.parametrize("dtype,C_in,C_out,N", CASES)
def test_forward(dtype, C_in, C_out, N, expanded, with_bias, cuda_device):
    print(f"[case] d4 {dtype} {C_in}->{C_out} N={N} expanded={expanded} bias={with_bias}", flush=True)
    x, W, b = make_inputs(8, C_in, C_out, N, dtype, seed=21)
    b = b if with_bias else None
    h = eq.prepare_weights(W.to(cuda_device), expanded=expanded, group="d4")
    fwd = eq.forward_expanded if expanded else eq.forward
    y = fwd(h, x.to(cuda_device), None if b is None else b.to(cuda_device))
    torch.cuda.synchronize()
    _check(y, d4.forward(x, W, b), dtype, f"d4 {dtype} {C_in}->{C_out} N={N} {'expanded' if expanded else 'spectral'} "
           f"[{h.describe()}]")


@pytest.mark.parametrize("w", D4_WORKLOADS, ids=[w.name for w in D4_WORKLOADS])
def test_full_size_all_tokens(w, cuda_device):
    print(f"[case] d4 full {w.name}", flush=True)
    x, W, b = make_inputs(w.G, w.C_in, w.C_out, w.N, w.dtype, seed=0)
    h = eq.prepare_weights(W.to(cuda_device), expanded=True, group="d4")
    xd, bd = x.to(cuda_device), b.to(cuda_device)
    outs = {"spectral": eq.forward(h, xd, bd), "expanded": eq.forward_expanded(h, xd, bd)}
    torch.cuda.synchronize()
    errs = compare_all_tokens(outs, lambda lo, hi: d4.forward(x[lo:hi], W, b), w.N, chunk=2048)
    for k, e in errs.items():
        print(f"[parity] {w.name} all {w.N} tokens {k}: rel_frob={e.rel:.3e} max_abs={e.max_abs:.3e}", flush=True)
        assert e.finite and e.rel <= REL_BF16 and e.max_abs <= MAX_BF16, (w.name, k, e.rel, e.max_abs)


@pytest.mark.parametrize("w", D4_WORKLOADS, ids=[w.name for w in D4_WORKLOADS])
def test_equivariance_under_rotation_and_reflection(w, cuda_device):
    # acting on the group axis of x by t (x'(g) = x(t^-1 g)) acts the same way on y; the transform's
    # coefficients are 0 and +-1, so the two runs see the same values up to signs and order
    x, W, b = make_inputs(w.G, w.C_in, w.C_out, 4096, w.dtype, seed=1)
    h = eq.prepare_weights(W.to(cuda_device), group="d4")
    xd, bd = x.to(cuda_device), b.to(cuda_device)
    y = eq.forward(h, xd, bd)
    for t in (1, 4, 5):  # r, s, r s
        perm = torch.as_tensor([d4.mul(d4.inv(t), g) for g in range(8)], device=cuda_device)
        yt = eq.forward(h, xd[:, :, perm].contiguous(), bd)
        torch.cuda.synchronize()
        diff = (yt.float() - y[:, :, perm].float()).abs().max().item()
        print(f"[equivariance] {w.name} t={t}: max |y(t.x) - t.y(x)| = {diff:.3e}", flush=True)
        assert diff <= 2e-2


def test_gelu_and_spectral_weights(cuda_device):
    x, W, b = make_inputs(8, 64, 128, 300, "bf16", seed=22)
    h = eq.prepare_weights(W.to(cuda_device), expanded=True, group="d4")
    y = eq.forward(h, x.to(cuda_device), b.to(cuda_device), act="gelu")
    ye = eq.forward_expanded(h, x.to(cuda_device), b.to(cuda_device), act="gelu")
    torch.cuda.synchronize()
    from oracle import gelu

    ref = gelu(d4.forward(x, W, b))
    _check(y, ref, "bf16", "d4 gelu spectral")
    _check(ye, ref, "bf16", "d4 gelu expanded")
    # stored spectral weights: the oracle's Fourier transform of W, to one bf16 rounding
    Wf = eq.export_spectral_weights(h).cpu().double().numpy()          # [8, C_out, C_in]
    ref_f = np.moveaxis(d4.fourier(W.double().numpy()), -1, 0)
    assert np.max(np.abs(Wf - ref_f) / np.maximum(np.abs(ref_f), 1e-3)) <= 2 ** -8
    # unrolled weight: exactly the group convolution's matrix
    E = eq.export_expanded_weight(h).cpu().double().numpy()
    np.testing.assert_array_equal(E, d4.expand(W.double().numpy()))


@pytest.mark.parametrize("dtype,C_in,C_out,N", [("bf16", 64, 64, 517), ("bf16", 64, 64, 30001),
                                                ("bf16", 32, 64, 1000), ("bf16", 256, 1024, 300),
                                                ("bf16", 192, 768, 2000),
                                                ("f32", 16, 24, 70)])
def test_backward(dtype, C_in, C_out, N, cuda_device):
    print(f"[case] d4 backward {dtype} {C_in}->{C_out} N={N}", flush=True)
    x, W, _ = make_inputs(8, C_in, C_out, N, dtype, seed=23)
    dy = make_grad(8, C_out, N, dtype, seed=23)
    h = eq.prepare_weights(W.to(cuda_device), backward=True, group="d4")
    dx = eq.backward_data(h, dy.to(cuda_device))
    dW, db = eq.backward_weights(h, x.to(cuda_device), dy.to(cuda_device))
    torch.cuda.synchronize()
    ref_dx = d4.backward_data(dy, W)
    ref_dW, ref_db = d4.backward_weights(x, dy)
    rms = lambda a: float(np.sqrt(np.mean(a * a)))
    _check(dx, ref_dx, dtype, f"d4 dx {dtype}", max_scale=rms(ref_dx))
    _check(dW, ref_dW, dtype, f"d4 dW {dtype}", max_scale=rms(ref_dW))
    _check(db, ref_db, dtype, f"d4 db {dtype}", max_scale=rms(ref_db))


def test_group_argument_errors(cuda_device):
    W = torch.zeros((8, 8, 4), dtype=torch.bfloat16, device=cuda_device)
    with pytest.raises(eq.EqlinError):
        eq.prepare_weights(W, group="d4")  # D4 needs G = 8
    with pytest.raises(ValueError):
        eq.prepare_weights(W, group="d8")
    W8 = torch.zeros((8, 8, 8), dtype=torch.bfloat16, device=cuda_device)
    h1 = eq.prepare_weights(W8, group="d4")
    h2 = eq.prepare_weights(W8)
    with pytest.raises(ValueError):  # a block cannot mix groups
        eq.mlp_block(h1, None, h2, None, torch.zeros((4, 8, 8), dtype=torch.bfloat16, device=cuda_device))
