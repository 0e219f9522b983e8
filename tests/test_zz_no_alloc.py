"""eqlin_backward_weights_static (no workspace, no allocation: the library's static per-device scratch)
against eqlin_backward_weights (caller workspace) through the C ABI.

Both run the same kernels on the same inputs, so the gradients must agree bit for bit; they are also
checked against the fp64 oracle with the gradient bars (bf16: relative Frobenius <= 1e-2 and max abs
<= 3e-2 * rms of the reference). Two calls in a row on each path, the second with fewer tokens: the
scratch keeps the first call's contents, which the second must not read.
"""
import ctypes

import numpy as np
import pytest
import torch

import fourier_domain_linear_amd as eq
import oracle
from fourier_domain_linear_amd.workloads import make_grad, make_inputs

pytestmark = pytest.mark.gpu

REL_BF16, MAX_BF16 = 1e-2, 3e-2


def _static(lib, h, xd, dyd, dW, db):
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.eqlin_backward_weights_static(ctypes.c_void_p(h.ptr), ctypes.c_void_p(xd.data_ptr()),
                                             ctypes.c_void_p(dyd.data_ptr()), ctypes.c_void_p(dW.data_ptr()),
                                             ctypes.c_void_p(db.data_ptr()), xd.shape[0], s)


def _workspace(lib, h, xd, dyd, dW, db, dev):
    N = xd.shape[0]
    need = lib.eqlin_backward_weights_workspace(ctypes.c_void_p(h.ptr), N)
    ws = torch.empty((max(1, need),), dtype=torch.uint8, device=dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.eqlin_backward_weights(ctypes.c_void_p(h.ptr), ctypes.c_void_p(xd.data_ptr()),
                                    ctypes.c_void_p(dyd.data_ptr()), ctypes.c_void_p(dW.data_ptr()),
                                    ctypes.c_void_p(db.data_ptr()), N, ctypes.c_void_p(ws.data_ptr()), need, s)
    torch.cuda.synchronize()
    return st


def _bar(got, ref, label):
    g = got.detach().to("cpu", torch.float64).numpy()
    d = g - ref
    rel = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
    rms = np.linalg.norm(ref) / np.sqrt(max(ref.size, 1))
    mx = float(np.max(np.abs(d)))
    print(f"[parity] {label}: rel_frob={rel:.3e} max_abs={mx:.3e} rms_ref={rms:.3e}", flush=True)
    assert np.all(np.isfinite(g)) and rel <= REL_BF16 and mx <= MAX_BF16 * rms, (label, rel, mx, rms)


# (G, C_in, C_out, first N, second N): the fused small-channel pass, and the three-pass
# large-channel path at token counts whose planes fit the static scratch
CASES = [(4, 96, 96, 25088, 3001), (8, 64, 64, 25088, 517), (8, 256, 1024, 500, 130), (4, 192, 768, 1000, 64)]


@pytest.mark.parametrize("G,C_in,C_out,N1,N2", CASES, ids=[f"p{c[0]}_{c[1]}x{c[2]}" for c in CASES])
def test_static_scratch_matches_workspace(G, C_in, C_out, N1, N2, cuda_device):
    lib = eq.load_library()
    x, W, _ = make_inputs(G, C_in, C_out, N1, "bf16", seed=17)
    dy = make_grad(G, C_out, N1, "bf16", seed=17)
    h = eq.prepare_weights(W.to(cuda_device))
    print(f"[case] static scratch G={G} {C_in}->{C_out} N={N1} then N={N2} [{h.describe()}]", flush=True)
    for N in (N1, N2):
        need = lib.eqlin_backward_weights_workspace(ctypes.c_void_p(h.ptr), N)
        assert 0 < need <= eq.STATIC_SCRATCH_BYTES, need
        xd, dyd = x[:N].contiguous().to(cuda_device), dy[:N].contiguous().to(cuda_device)
        dW_s = torch.full((C_out, C_in, G), float("nan"), dtype=torch.float32, device=cuda_device)
        db_s = torch.full((C_out,), float("nan"), dtype=torch.float32, device=cuda_device)
        assert _static(lib, h, xd, dyd, dW_s, db_s) == eq.EQLIN_OK, lib.eqlin_last_error()
        torch.cuda.synchronize()
        dW_w = torch.empty_like(dW_s)
        db_w = torch.empty_like(db_s)
        assert _workspace(lib, h, xd, dyd, dW_w, db_w, cuda_device) == eq.EQLIN_OK
        assert torch.equal(dW_s, dW_w) and torch.equal(db_s, db_w), f"N={N}: static and workspace paths differ"
        rW, rb = oracle.backward_weights(x[:N], dy[:N])
        _bar(dW_s, rW, f"static dW G={G} {C_in}->{C_out} N={N}")
        _bar(db_s, rb, f"static db G={G} {C_in}->{C_out} N={N}")


def test_static_scratch_rejects_oversize_and_takes_empty(cuda_device):
    lib = eq.load_library()
    G, C_in, C_out = 8, 256, 1024
    N = 12544  # the three-pass path's planes and partials need far more than the static array
    x, W, _ = make_inputs(G, C_in, C_out, N, "bf16", seed=18)
    dy = make_grad(G, C_out, N, "bf16", seed=18)
    h = eq.prepare_weights(W.to(cuda_device))
    assert lib.eqlin_backward_weights_workspace(ctypes.c_void_p(h.ptr), N) > eq.STATIC_SCRATCH_BYTES
    xd, dyd = x.to(cuda_device), dy.to(cuda_device)
    dW = torch.full((C_out, C_in, G), 7.0, dtype=torch.float32, device=cuda_device)
    db = torch.full((C_out,), 7.0, dtype=torch.float32, device=cuda_device)
    assert _static(lib, h, xd, dyd, dW, db) == eq.EQLIN_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((dW == 7.0).all()) and bool((db == 7.0).all())  # nothing enqueued
    # no tokens: zero gradients, no scratch
    assert _static(lib, h, xd[:0], dyd[:0], dW, db) == eq.EQLIN_OK
    torch.cuda.synchronize()
    assert bool((dW == 0).all()) and bool((db == 0).all())
