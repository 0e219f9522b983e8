"""GPU parity of the backward passes (eqlin_backward_data, eqlin_backward_weights) through the C ABI
against the fp64 oracle's gradients (oracle.backward_data / oracle.backward_weights) on the same
seeded bf16-rounded inputs.

Bars. The forward's bars are stated for outputs of unit scale; the gradients are not (dx has rms
sqrt(C_out / C_in) here, dW grows like sqrt(N)), so the max-abs bar is taken relative to the
reference's rms: bf16 -- relative Frobenius error <= 1e-2 AND max abs error <= 3e-2 * rms(ref);
fp32 -- relative Frobenius error <= 1e-5. (For the forward's unit-scale outputs this is the forward's
own bar.)

Sizes: small ragged shapes the oracle finishes in seconds (several tiles, partial token steps,
padded channels), and every workload's channel shape at its full token count with every element
compared: dx over all tokens (the oracle streamed over token chunks), dW and db over all channels and
all tokens.
"""
import numpy as np
import pytest
import torch

import fourier_domain_linear_amd as eq
import oracle
from fourier_domain_linear_amd.workloads import WORKLOADS, make_grad, make_inputs
from fullsize import compare_all_tokens

pytestmark = pytest.mark.gpu

REL_BF16, MAX_BF16, REL_F32 = 1e-2, 3e-2, 1e-5


def _check(got: torch.Tensor, ref: np.ndarray, dtype: str, label: str):
    g = got.detach().to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(g)), label
    diff = g - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / max(nref, 1e-300)
    rms = nref / np.sqrt(max(ref.size, 1))
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    print(f"[parity] {label}: rel_frob={rel:.3e} max_abs={mx:.3e} rms_ref={rms:.3e}", flush=True)
    if dtype == "bf16":
        assert rel <= REL_BF16 and mx <= MAX_BF16 * max(rms, 1e-30), (label, rel, mx, rms)
    else:
        assert rel <= REL_F32, (label, rel)


def _handle(W, dev):
    return eq.prepare_weights(W.to(dev), backward=True)


SHAPES = [(4, 32, 48, 1000, "bf16"), (8, 64, 64, 517, "bf16"), (4, 96, 96, 777, "bf16"),
          (4, 192, 768, 300, "bf16"), (8, 256, 1024, 130, "bf16"), (8, 136, 200, 203, "bf16"),
          (4, 40, 24, 70, "bf16"), (2, 64, 32, 333, "bf16"), (1, 48, 40, 100, "bf16"),
          (4, 16, 16, 64, "f32"), (8, 24, 40, 150, "f32")]


@pytest.mark.parametrize("G,C_in,C_out,N,dtype", SHAPES,
                         ids=[f"p{g}_{ci}x{co}_n{n}_{d}" for g, ci, co, n, d in SHAPES])
def test_backward_small(G, C_in, C_out, N, dtype, cuda_device):
    x, W, _ = make_inputs(G, C_in, C_out, N, dtype, seed=11)
    dy = make_grad(G, C_out, N, dtype, seed=11)
    h = _handle(W, cuda_device)
    dx = eq.backward_data(h, dy.to(cuda_device))
    dW, db = eq.backward_weights(h, x.to(cuda_device), dy.to(cuda_device))
    torch.cuda.synchronize()
    print(f"[kernel] {h.describe()}", flush=True)
    _check(dx, oracle.backward_data(dy, W), dtype, f"dx G={G} {C_in}x{C_out} N={N} {dtype}")
    rW, rb = oracle.backward_weights(x, dy)
    _check(dW, rW, dtype, f"dW G={G} {C_in}x{C_out} N={N} {dtype}")
    _check(db, rb, dtype, f"db G={G} {C_in}x{C_out} N={N} {dtype}")


@pytest.mark.parametrize("w", WORKLOADS, ids=[w.name for w in WORKLOADS])
def test_backward_full_size_all(w, cuda_device):
    # every element of dx (all tokens, streamed over token chunks) and of dW, db (all channels, all
    # tokens), in the configuration the benchmark's --backward leg runs
    x, W, _ = make_inputs(w.G, w.C_in, w.C_out, w.N, w.dtype, seed=0)
    dy = make_grad(w.G, w.C_out, w.N, w.dtype, seed=0)
    h = _handle(W, cuda_device)
    xd, dyd = x.to(cuda_device), dy.to(cuda_device)
    dx = eq.backward_data(h, dyd)
    dW, db = eq.backward_weights(h, xd, dyd)
    torch.cuda.synchronize()
    print(f"[kernel] {h.describe()}", flush=True)
    e = compare_all_tokens({"dx": dx}, lambda lo, hi: oracle.backward_data(dy[lo:hi], W), w.N, chunk=2048)["dx"]
    print(f"[parity] {w.name} dx all {w.N} tokens: rel_frob={e.rel:.3e} max_abs={e.max_abs:.3e} "
          f"rms_ref={e.rms:.3e}", flush=True)
    assert e.finite
    if w.dtype == "bf16":
        assert e.rel <= REL_BF16 and e.max_abs <= MAX_BF16 * e.rms, (w.name, e.rel, e.max_abs, e.rms)
    else:
        assert e.rel <= REL_F32, (w.name, e.rel)
    rW, rb = oracle.backward_weights(x, dy)
    _check(dW, rW, w.dtype, f"{w.name} dW all channels, all {w.N} tokens")
    _check(db, rb, w.dtype, f"{w.name} db all channels")


@pytest.mark.parametrize("G,C,N", [(8, 64, 70001), (4, 96, 50003)])
def test_backward_weights_long_token_ranges(G, C, N, cuda_device):
    # several 64-token super-chunks per workgroup and a ragged last range (the fused small-channel pass)
    x, W, _ = make_inputs(G, C, C, N, "bf16", seed=13)
    dy = make_grad(G, C, N, "bf16", seed=13)
    h = _handle(W, cuda_device)
    dW, db = eq.backward_weights(h, x.to(cuda_device), dy.to(cuda_device))
    torch.cuda.synchronize()
    print(f"[kernel] {h.describe()}", flush=True)
    rW, rb = oracle.backward_weights(x, dy)
    _check(dW, rW, "bf16", f"dW G={G} C={C} N={N} all channels")
    _check(db, rb, "bf16", f"db G={G} C={C} N={N}")


def test_backward_weights_empty_and_tiny(cuda_device):
    x, W, _ = make_inputs(8, 32, 64, 1, "bf16", seed=5)
    h = _handle(W, cuda_device)
    dW, db = eq.backward_weights(h, x[:0].to(cuda_device), make_grad(8, 64, 0).to(cuda_device))
    assert torch.count_nonzero(dW).item() == 0 and torch.count_nonzero(db).item() == 0
    dy = make_grad(8, 64, 1, seed=5)
    dW, db = eq.backward_weights(h, x.to(cuda_device), dy.to(cuda_device))
    rW, rb = oracle.backward_weights(x, dy)
    _check(dW, rW, "bf16", "dW N=1")
    _check(db, rb, "bf16", "db N=1")
    assert eq.backward_data(h, dy[:0].to(cuda_device)).shape == (0, 32, 8)


def test_backward_without_bias_and_reused_workspace(cuda_device):
    x, W, _ = make_inputs(4, 64, 128, 2000, "bf16", seed=9)
    dy = make_grad(4, 128, 2000, seed=9)
    h = _handle(W, cuda_device)
    need = eq.backward_weights_workspace(h, 2000)
    ws = torch.empty((need,), dtype=torch.uint8, device=cuda_device)
    ws.fill_(0xff)  # garbage in the workspace must not leak into the result
    dW1, db1 = eq.backward_weights(h, x.to(cuda_device), dy.to(cuda_device), with_bias=False, workspace=ws)
    assert db1 is None
    dW2, _ = eq.backward_weights(h, x[:700].to(cuda_device), dy[:700].to(cuda_device), workspace=ws)
    torch.cuda.synchronize()
    _check(dW1, oracle.backward_weights(x, dy)[0], "bf16", "dW N=2000 caller workspace")
    _check(dW2, oracle.backward_weights(x[:700], dy[:700])[0], "bf16", "dW N=700 same workspace")


def test_backward_data_needs_flag(cuda_device):
    _, W, _ = make_inputs(4, 32, 32, 1, "bf16")
    h = eq.prepare_weights(W.to(cuda_device))
    with pytest.raises(ValueError):
        eq.backward_data(h, make_grad(4, 32, 4).to(cuda_device))


def test_backward_bf16_needs_c_out_multiple_of_8(cuda_device):
    _, W, _ = make_inputs(4, 32, 12, 1, "bf16")
    with pytest.raises(eq.EqlinError) as ei:
        eq.prepare_weights(W.to(cuda_device), backward=True)
    assert ei.value.status == eq.EQLIN_ERR_UNSUPPORTED


@pytest.mark.parametrize("w", WORKLOADS, ids=[w.name for w in WORKLOADS])
def test_backward_data_expanded_full_size(w, cuda_device):
    # the naive comparator of dx (one dense product with the unrolled weight), every token
    x, W, _ = make_inputs(w.G, w.C_in, w.C_out, w.N, w.dtype, seed=0)
    dy = make_grad(w.G, w.C_out, w.N, w.dtype, seed=0)
    h = eq.prepare_weights(W.to(cuda_device), expanded=True, backward=True)
    dx = eq.backward_data_expanded(h, dy.to(cuda_device))
    torch.cuda.synchronize()
    e = compare_all_tokens({"dx": dx}, lambda lo, hi: oracle.backward_data(dy[lo:hi], W), w.N, chunk=2048)["dx"]
    print(f"[parity] {w.name} expanded dx all {w.N} tokens: rel_frob={e.rel:.3e} max_abs={e.max_abs:.3e} "
          f"rms_ref={e.rms:.3e}", flush=True)
    assert e.finite
    if w.dtype == "bf16":
        assert e.rel <= REL_BF16 and e.max_abs <= MAX_BF16 * e.rms, (w.name, e.rel, e.max_abs, e.rms)
    else:
        assert e.rel <= REL_F32, (w.name, e.rel)


@pytest.mark.parametrize("G,C_in,C_out,N", [(4, 40, 24, 70), (8, 136, 200, 203), (2, 64, 32, 333), (1, 48, 40, 100)])
def test_backward_data_expanded_small(G, C_in, C_out, N, cuda_device):
    x, W, _ = make_inputs(G, C_in, C_out, N, "bf16", seed=12)
    dy = make_grad(G, C_out, N, "bf16", seed=12)
    h = eq.prepare_weights(W.to(cuda_device), expanded=True, backward=True)
    dx = eq.backward_data_expanded(h, dy.to(cuda_device))
    torch.cuda.synchronize()
    _check(dx, oracle.backward_data(dy, W), "bf16", f"expanded dx G={G} {C_in}x{C_out} N={N}")
    # without EQLIN_PREPARE_EXPANDED the entry point refuses
    import ctypes

    h2 = eq.prepare_weights(W.to(cuda_device), backward=True)
    dyd = dy.to(cuda_device)
    st = eq.load_library().eqlin_backward_data_expanded(
        ctypes.c_void_p(h2.ptr), ctypes.c_void_p(dyd.data_ptr()), ctypes.c_void_p(dx.data_ptr()), N,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == eq.EQLIN_ERR_INVALID_ARG
