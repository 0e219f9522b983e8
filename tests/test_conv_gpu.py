"""GPU parity of the p4 group convolution with k x k kernels (eqlin_prepare_conv_weights,
eqlin_conv_forward, eqlin_conv_forward_expanded) against the fp64 oracle (oracle/conv.py) on the same
seeded bf16-rounded inputs.

The library runs the convolution as an EQ-Linear layer over C_in * k^2 gathered channels (each
gathered sample read from a rotated neighbour pixel while loading x), through the same spectral
kernel as the layer; the expanded comparator runs the same gathered layer as one dense product.

Bars: the layer's -- bf16: relative Frobenius error <= 1e-2 AND max abs error <= 3e-2 (the inputs'
variances give outputs of about unit scale, as for the layer); fp16: the bf16 bars / 8.
Sizes: small images with ragged token counts (several tiles, a partial one, images smaller than the
filter, one-pixel images), k = 1, 3, 5, 7, 9, C_out not a multiple of the output tile, C_in / 16 not a
multiple of 4 (the centre's last group part filling); and the benchmark's shape at full size with
every output compared.
"""
import ctypes

import numpy as np
import pytest
import torch

import fourier_domain_linear_amd as eq
import oracle
from fourier_domain_linear_amd.workloads import CONV_WORKLOAD, make_conv_inputs
from fullsize import compare_all_tokens
from oracle import conv

pytestmark = pytest.mark.gpu

REL_BF16, MAX_BF16 = 1e-2, 3e-2


def _check(y_gpu, ref, label, dtype="bf16"):
    y = y_gpu.detach().to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(y)), label
    d = y - ref
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(d))) if d.size else 0.0
    print(f"[parity] {label}: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    scale = 1.0 if dtype == "bf16" else 1.0 / 8
    assert rel <= REL_BF16 * scale and mx <= MAX_BF16 * scale, (label, rel, mx)


CASES = [  # B, H, W, C_in, C_out, k
    (2, 9, 7, 16, 8, 3), (1, 12, 12, 32, 256, 3), (3, 5, 6, 16, 264, 5), (1, 1, 1, 16, 8, 3),
    (2, 17, 19, 48, 296, 3), (1, 6, 6, 64, 512, 1), (4, 2, 3, 16, 16, 5), (1, 30, 31, 32, 64, 3),
    (2, 7, 9, 80, 40, 3), (1, 8, 5, 48, 24, 5), (1, 9, 10, 32, 16, 7), (1, 5, 4, 16, 8, 9)]


@pytest.mark.parametrize("with_bias", [True, False], ids=["bias", "nobias"])
@pytest.mark.parametrize("B,H,W,C_in,C_out,k", CASES, ids=[f"b{c[0]}_{c[1]}x{c[2]}_c{c[3]}x{c[4]}_k{c[5]}" for c in CASES])
def test_conv_small(B, H, W, C_in, C_out, k, with_bias, cuda_device):
    x, psi, b = make_conv_inputs(C_in, C_out, k, B, H, W, "bf16", seed=B * 100 + k)
    b = b if with_bias else None
    h = eq.prepare_conv_weights(psi.to(cuda_device), expanded=True)
    print(f"[case] conv {B}x{H}x{W} {C_in}->{C_out} k={k} bias={with_bias} [{h.describe()}]", flush=True)
    xd, bd = x.to(cuda_device), None if b is None else b.to(cuda_device)
    y = eq.conv_forward(h, xd, bd)
    ye = eq.conv_forward_expanded(h, xd, bd)
    torch.cuda.synchronize()
    ref = conv.forward(x, psi, b)
    _check(y, ref, f"conv {B}x{H}x{W} {C_in}->{C_out} k={k} spectral")
    _check(ye, ref, f"conv {B}x{H}x{W} {C_in}->{C_out} k={k} expanded")


def test_conv_k1_is_the_layer(cuda_device):
    # a 1 x 1 group convolution is the EQ-Linear layer on one token per pixel
    x, psi, b = make_conv_inputs(32, 48, 1, 2, 11, 13, "bf16", seed=5)
    h = eq.prepare_conv_weights(psi.to(cuda_device))
    y = eq.conv_forward(h, x.to(cuda_device), b.to(cuda_device))
    hl = eq.prepare_weights(psi[..., 0, 0].contiguous().to(cuda_device))
    yl = eq.forward(hl, x.reshape(-1, 32, 4).to(cuda_device), b.to(cuda_device))
    torch.cuda.synchronize()
    ref = oracle.forward(x.reshape(-1, 32, 4), psi[..., 0, 0], b)
    _check(y.reshape(-1, 48, 4), ref, "conv k=1 vs the layer's oracle")
    _check(yl, ref, "layer on the same tokens")


def test_conv_f16(cuda_device):
    x, psi, b = make_conv_inputs(32, 256, 3, 2, 10, 9, "f16", seed=6)
    h = eq.prepare_conv_weights(psi.to(cuda_device), expanded=True)
    xd, bd = x.to(cuda_device), b.to(cuda_device)
    y, ye = eq.conv_forward(h, xd, bd), eq.conv_forward_expanded(h, xd, bd)
    torch.cuda.synchronize()
    assert y.dtype == torch.float16
    ref = conv.forward(x, psi, b)
    _check(y, ref, "conv f16 spectral", "f16")
    _check(ye, ref, "conv f16 expanded", "f16")


def test_conv_equivariance_on_gpu(cuda_device):
    # quarter turn of the image plus a group shift commutes with the layer; here on the GPU's own
    # outputs (holds at any size, bounded by the rounding of the two results)
    x, psi, b = make_conv_inputs(32, 256, 3, 2, 24, 24, "bf16", seed=7)
    h = eq.prepare_conv_weights(psi.to(cuda_device))
    xd, bd = x.to(cuda_device), b.to(cuda_device)
    y = eq.conv_forward(h, xd, bd).double()
    for m in (1, 2, 3):
        xt = torch.roll(torch.rot90(xd, m, dims=(1, 2)), m, dims=4).contiguous()
        yt = eq.conv_forward(h, xt, bd).double()
        ref = torch.roll(torch.rot90(y, m, dims=(1, 2)), m, dims=4)
        rel = (torch.linalg.vector_norm(yt - ref) / torch.linalg.vector_norm(ref)).item()
        print(f"[equivariance] conv turn={m} rel={rel:.3e}", flush=True)
        assert rel <= 1e-2


def test_conv_full_size_all_tokens(cuda_device):
    w = CONV_WORKLOAD
    x, psi, b = make_conv_inputs(w.C_in, w.C_out, w.k, w.B, w.H, w.W, w.dtype, seed=0)
    h = eq.prepare_conv_weights(psi.to(cuda_device), expanded=True)
    print(f"[case] conv full {w.name} [{h.describe()}]", flush=True)
    xd, bd = x.to(cuda_device), b.to(cuda_device)
    outs = {"spectral": eq.conv_forward(h, xd, bd).reshape(w.N, w.C_out, 4),
            "expanded": eq.conv_forward_expanded(h, xd, bd).reshape(w.N, w.C_out, 4)}
    torch.cuda.synchronize()
    # the oracle image by image (one image's pixels are one chunk of tokens)
    per = w.H * w.W
    errs = compare_all_tokens(outs, lambda lo, hi: conv.forward(x[lo // per:hi // per], psi, b).reshape(-1, w.C_out, 4),
                              w.N, chunk=per)
    for k, e in errs.items():
        print(f"[parity] {w.name} all {w.N} pixels {k}: rel_frob={e.rel:.3e} max_abs={e.max_abs:.3e}", flush=True)
        assert e.finite and e.rel <= REL_BF16 and e.max_abs <= MAX_BF16, (k, e.rel, e.max_abs)


def test_conv_argument_errors(cuda_device):
    lib = eq.load_library()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    _, psi, _ = make_conv_inputs(16, 8, 3, 1, 1, 1, "bf16")
    pd = psi.to(cuda_device)
    out = ctypes.c_void_p()
    P = ctypes.c_void_p(pd.data_ptr())
    # G must be 4, k odd, C_in a multiple of 16, C_out a multiple of 8
    assert lib.eqlin_prepare_conv_weights(P, 8, 16, 8, 3, eq.EQLIN_BF16, 0, s, ctypes.byref(out)) == eq.EQLIN_ERR_INVALID_ARG
    assert lib.eqlin_prepare_conv_weights(P, 8, 16, 4, 2, eq.EQLIN_BF16, 0, s, ctypes.byref(out)) == eq.EQLIN_ERR_INVALID_ARG
    assert lib.eqlin_prepare_conv_weights(P, 8, 8, 4, 3, eq.EQLIN_BF16, 0, s, ctypes.byref(out)) == eq.EQLIN_ERR_UNSUPPORTED
    assert lib.eqlin_prepare_conv_weights(P, 4, 16, 4, 3, eq.EQLIN_BF16, 0, s, ctypes.byref(out)) == eq.EQLIN_ERR_UNSUPPORTED
    assert lib.eqlin_prepare_conv_weights(P, 8, 16, 4, 3, eq.EQLIN_F32, 0, s, ctypes.byref(out)) == eq.EQLIN_ERR_UNSUPPORTED
    assert lib.eqlin_prepare_conv_weights(P, 8, 16, 4, 3, eq.EQLIN_BF16, eq.EQLIN_PREPARE_BACKWARD, s,
                                          ctypes.byref(out)) == eq.EQLIN_ERR_UNSUPPORTED
    h = eq.prepare_conv_weights(pd)
    x = torch.zeros((2, 3, 5, 16, 4), dtype=torch.bfloat16, device=cuda_device)
    y = torch.empty((2, 3, 5, 8, 4), dtype=torch.bfloat16, device=cuda_device)
    X, Y, H = ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(h.ptr)
    assert lib.eqlin_conv_forward(H, X, None, Y, 2, 3, 5, s) == eq.EQLIN_OK
    assert lib.eqlin_conv_forward(H, X, None, Y, -1, 3, 5, s) == eq.EQLIN_ERR_INVALID_ARG
    assert lib.eqlin_conv_forward(H, X, None, Y, 2, 3, 0, s) == eq.EQLIN_OK  # empty image: nothing to do
    # a batch whose x would span more than 2^31 bytes is refused on the host before any launch (with
    # these small buffers the extents that size implies overlap y, which is checked first; the
    # buffers are never touched)
    assert lib.eqlin_conv_forward(H, X, None, Y, 5000, 64, 64, s) in (eq.EQLIN_ERR_INVALID_ARG,
                                                                      eq.EQLIN_ERR_UNSUPPORTED)
    # a convolution handle is not a layer handle, and the other way round
    assert lib.eqlin_forward(H, X, None, Y, 30, s) == eq.EQLIN_ERR_INVALID_ARG
    assert lib.eqlin_conv_forward_expanded(H, X, None, Y, 2, 3, 5, s) == eq.EQLIN_ERR_INVALID_ARG  # no EXPANDED flag
    _, W, _ = make_conv_inputs(16, 8, 1, 1, 1, 1, "bf16")
    hl = eq.prepare_weights(W[..., 0, 0].contiguous().to(cuda_device))
    assert lib.eqlin_conv_forward(ctypes.c_void_p(hl.ptr), X, None, Y, 2, 3, 5, s) == eq.EQLIN_ERR_INVALID_ARG
    torch.cuda.synchronize()
