"""GPU parity of the fused activation and of the transformer MLP block built on the layer.

The block is EQ-Linear(C -> 4C), GELU, EQ-Linear(4C -> C), the MLP of the transformer stages the
layer is integrated into ("Flash EQ-Linear" explainer, "Resultados Experimentales", network level);
GELU is the exact form x * Phi(x) (the ViT-on-mobile page names the activation, "El Efecto GELU").
On the GPU the GELU runs in the first layer's epilogue (eqlin_forward_act), the hidden activation
is stored once in the layer's dtype, and the second layer reads it.

Bars: those of the layer itself -- bf16: relative Frobenius error <= 1e-2 AND max abs error <= 3e-2
against the fp64 oracle fed the same bf16-rounded inputs (the oracle keeps the hidden activation in
fp64, so the block's bar also covers the one bf16 rounding of the hidden layer); fp32: relative
Frobenius error <= 1e-5.
"""
import ctypes

import numpy as np
import pytest
import torch

import fourier_domain_linear_amd as eq
import oracle
from fourier_domain_linear_amd.workloads import BLOCK_WORKLOAD, make_block_inputs, make_inputs
from fullsize import compare_all_tokens

pytestmark = pytest.mark.gpu

REL_BF16, MAX_BF16, REL_F32 = 1e-2, 3e-2, 1e-5


def _check(y_gpu, ref, dtype, label):
    y = y_gpu.detach().to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(y)), label
    diff = y - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    print(f"[parity] {label}: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    if dtype == "bf16":
        assert rel <= REL_BF16 and mx <= MAX_BF16, (label, rel, mx)
    else:
        assert rel <= REL_F32, (label, rel)


# Shapes that reach every forward kernel family and both store paths: the streaming kernel (G = 4, 8,
# 2, 1; whole and partial 16-output blocks), the large-channel kernels (G = 4; G = 8 with the plane
# split; whole rows and element stores for C_out * G % 8 != 0), and the fp32 kernel.
ACT_CASES = [
    ("bf16", 4, 96, 96, 517), ("bf16", 8, 64, 64, 517), ("bf16", 2, 64, 72, 300), ("bf16", 1, 64, 40, 300),
    ("bf16", 4, 40, 20, 130), ("bf16", 4, 192, 768, 517), ("bf16", 8, 256, 1024, 300),
    ("bf16", 4, 128, 4095, 200), ("bf16", 4, 768, 192, 300),
    ("f32", 4, 16, 16, 64), ("f32", 8, 24, 40, 77), ("f32", 1, 32, 8, 50),
]


@pytest.mark.parametrize("expanded", [False, True], ids=["spectral", "expanded"])
@pytest.mark.parametrize("dtype,G,C_in,C_out,N", ACT_CASES)
def test_forward_gelu(dtype, G, C_in, C_out, N, expanded, cuda_device):
    print(f"[case] gelu {dtype} G={G} C_in={C_in} C_out={C_out} N={N} expanded={expanded}", flush=True)
    x, W, b = make_inputs(G, C_in, C_out, N, dtype, seed=3)
    h = eq.prepare_weights(W.to(cuda_device), expanded=expanded)
    fwd = eq.forward_expanded if expanded else eq.forward
    y = fwd(h, x.to(cuda_device), b.to(cuda_device), act="gelu")
    torch.cuda.synchronize()
    _check(y, oracle.gelu(oracle.forward(x, W, b)), dtype,
           f"gelu {dtype} G={G} {C_in}->{C_out} N={N} {'expanded' if expanded else 'spectral'} [{h.describe()}]")


@pytest.mark.parametrize("dtype,G", [("f32", 4), ("bf16", 4), ("bf16", 8)])
def test_forward_gelu_wide_range(dtype, G, cuda_device):
    # outputs spread over about +-100: the far tails (GELU -> 0 for v << 0, -> v for v >> 0) and the
    # transition, all against the oracle's erf
    x, W, b = make_inputs(G, 64, 64, 200, dtype, seed=9)
    x = (x.float() * 25).to(x.dtype)
    h = eq.prepare_weights(W.to(cuda_device))
    y = eq.forward(h, x.to(cuda_device), b.to(cuda_device), act="gelu")
    torch.cuda.synchronize()
    pre = oracle.forward(x, W, b)
    assert pre.max() > 40 and pre.min() < -40
    ref = oracle.gelu(pre)
    if dtype == "bf16":  # the bar's max-abs term is for unit-scale outputs: scale it with the output
        yv = y.to("cpu", torch.float64).numpy()
        rel = np.linalg.norm(yv - ref) / np.linalg.norm(ref)
        assert rel <= REL_BF16 and np.max(np.abs(yv - ref)) <= MAX_BF16 * np.abs(pre).max() / 3, rel
        neg = pre < -10  # deep negative tail: exactly representable tiny values, no sign flips
        assert np.all(np.abs(yv[neg]) <= 1e-6)
    else:
        _check(y, ref, dtype, f"gelu wide range {dtype} G={G}")


def test_forward_gelu_no_bias_and_plain_unchanged(cuda_device):
    # act = none through eqlin_forward_act is eqlin_forward, bit for bit (the same kernel); GELU with
    # no bias against the oracle.
    x, W, _ = make_inputs(4, 192, 768, 333, "bf16", seed=5)
    h = eq.prepare_weights(W.to(cuda_device))
    xd = x.to(cuda_device)
    y_plain = eq.forward(h, xd)
    y_none = torch.empty_like(y_plain)
    lib = eq.load_library()
    st = lib.eqlin_forward_act(ctypes.c_void_p(h.ptr), ctypes.c_void_p(xd.data_ptr()), None,
                               ctypes.c_void_p(y_none.data_ptr()), 333, eq.EQLIN_ACT_NONE, None)
    assert st == eq.EQLIN_OK
    y_gelu = eq.forward(h, xd, act="gelu")
    torch.cuda.synchronize()
    assert torch.equal(y_plain, y_none)
    _check(y_gelu, oracle.gelu(oracle.forward(x, W)), "bf16", "gelu no bias")


def test_unknown_activation_rejected(cuda_device):
    x, W, b = make_inputs(4, 32, 32, 16, "bf16", seed=6)
    h = eq.prepare_weights(W.to(cuda_device), expanded=True)
    xd, y = x.to(cuda_device), torch.zeros((16, 32, 4), dtype=torch.bfloat16, device=cuda_device)
    lib = eq.load_library()
    for fn in (lib.eqlin_forward_act, lib.eqlin_forward_expanded_act):
        for act in (-1, 2, 99):
            st = fn(ctypes.c_void_p(h.ptr), ctypes.c_void_p(xd.data_ptr()), None, ctypes.c_void_p(y.data_ptr()),
                    16, act, None)
            assert st == eq.EQLIN_ERR_INVALID_ARG
            assert "activation" in lib.eqlin_last_error().decode()
    torch.cuda.synchronize()
    assert not y.any()  # nothing was enqueued
    with pytest.raises(ValueError):
        eq.forward(h, xd, act="relu")


def _block(dev, x, W1, b1, W2, b2, expanded):
    h1 = eq.prepare_weights(W1.to(dev), expanded=expanded)
    h2 = eq.prepare_weights(W2.to(dev), expanded=expanded)
    y = eq.mlp_block(h1, b1.to(dev), h2, b2.to(dev), x.to(dev), expanded=expanded)
    torch.cuda.synchronize()
    return y, h1, h2


@pytest.mark.parametrize("expanded", [False, True], ids=["spectral", "expanded"])
@pytest.mark.parametrize("dtype,G,C,N", [("bf16", 4, 64, 517), ("bf16", 8, 64, 300), ("bf16", 4, 192, 300),
                                         ("bf16", 2, 32, 100), ("f32", 4, 16, 64), ("f32", 8, 16, 33)])
def test_mlp_block_small(dtype, G, C, N, expanded, cuda_device):
    print(f"[case] block {dtype} G={G} C={C} N={N} expanded={expanded}", flush=True)
    x, W1, b1, W2, b2 = make_block_inputs(G, C, 4 * C, N, dtype, seed=7)
    y, h1, h2 = _block(cuda_device, x, W1, b1, W2, b2, expanded)
    _check(y, oracle.mlp_block(x, W1, b1, W2, b2), dtype,
           f"block {dtype} G={G} C={C} N={N} {'expanded' if expanded else 'spectral'} [{h1.describe()} / {h2.describe()}]")


@pytest.mark.parametrize("expanded", [False, True], ids=["spectral", "expanded"])
def test_mlp_block_full_size_all_tokens(expanded, cuda_device):
    w = BLOCK_WORKLOAD
    print(f"[case] block full {w.name} expanded={expanded}", flush=True)
    x, W1, b1, W2, b2 = make_block_inputs(w.G, w.C_in, w.C_out, w.N, w.dtype, seed=0)
    y, _, _ = _block(cuda_device, x, W1, b1, W2, b2, expanded)
    e = compare_all_tokens({"y": y}, lambda lo, hi: oracle.mlp_block(x[lo:hi], W1, b1, W2, b2), w.N,
                           chunk=2048)["y"]
    print(f"[parity] block {w.name} all {w.N} tokens {'expanded' if expanded else 'spectral'}: "
          f"rel_frob={e.rel:.3e} max_abs={e.max_abs:.3e}", flush=True)
    assert e.finite and e.rel <= REL_BF16 and e.max_abs <= MAX_BF16, (e.rel, e.max_abs)


def test_mlp_block_empty_and_one_token(cuda_device):
    x, W1, b1, W2, b2 = make_block_inputs(4, 32, 128, 1, "bf16", seed=8)
    y, h1, h2 = _block(cuda_device, x, W1, b1, W2, b2, False)
    _check(y, oracle.mlp_block(x, W1, b1, W2, b2), "bf16", "block N=1")
    y0 = eq.mlp_block(h1, b1.to(cuda_device), h2, b2.to(cuda_device), x[:0].to(cuda_device))
    assert tuple(y0.shape) == (0, 32, 4)


def test_block_graph_replay_matches_eager(cuda_device):
    # the block (two launches, GELU in the first) captured in one HIP graph: every replay equals the
    # eager result, with unrelated eager work and synchronisations between replays; D4 and fp16 too
    for group, dtype, G in (("cyclic", "bf16", 4), ("d4", "bf16", 8), ("cyclic", "f16", 4)):
        x, W1, b1, W2, b2 = make_block_inputs(G, 64, 256, 1000, dtype, seed=12)
        h1 = eq.prepare_weights(W1.to(cuda_device), group=group)
        h2 = eq.prepare_weights(W2.to(cuda_device), group=group)
        xd, b1d, b2d = x.to(cuda_device), b1.to(cuda_device), b2.to(cuda_device)
        ref = eq.mlp_block(h1, b1d, h2, b2d, xd)
        hid = torch.empty((1000, 256, G), dtype=ref.dtype, device=cuda_device)
        y = torch.empty_like(ref)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            eq.mlp_block(h1, b1d, h2, b2d, xd, hid, y)
        for r in range(3):
            y.fill_(float("nan"))
            eq.forward(h1, xd, None, act="gelu")  # unrelated eager work
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, ref), (group, dtype, r)
