"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs.

Bars (fixed up front for this layer): bf16 path -- relative Frobenius error <= 1e-2 AND max abs
error <= 3e-2 against the unrounded fp64 oracle fed the same bf16-rounded x, W, b; fp32 path --
relative Frobenius error <= 1e-5. The oracle is exact arithmetic (fp64) of the unrolled layer, so
any correct fast path lands within rounding of it ("Flash EQ-Linear" explainer, "Principales
Contribuciones": the method is exact up to floating point).

Sizes: every workload's channel shape at a ragged token count the oracle finishes in seconds
(several tiles plus a partial one), and every workload at its full token count, every token compared
(the oracle streamed over token chunks), in the same launch configuration the benchmark times.
"""
import ctypes

import numpy as np
import pytest
import torch

import fourier_domain_linear_amd as eq
import oracle
from fourier_domain_linear_amd.workloads import WORKLOADS, make_inputs
from fullsize import compare_all_tokens

pytestmark = pytest.mark.gpu

REL_BF16, MAX_BF16, REL_F32 = 1e-2, 3e-2, 1e-5


def _errors(y_gpu: torch.Tensor, ref: np.ndarray):
    y = y_gpu.detach().to("cpu", torch.float64).numpy()
    diff = y - ref
    rel = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)
    return float(rel), float(np.max(np.abs(diff))) if diff.size else 0.0


def _check(y_gpu, ref, dtype: str, label: str):
    rel, mx = _errors(y_gpu, ref)
    print(f"[parity] {label}: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert np.all(np.isfinite(y_gpu.detach().float().cpu().numpy())), label
    if dtype == "bf16":
        assert rel <= REL_BF16 and mx <= MAX_BF16, (label, rel, mx)
    else:
        assert rel <= REL_F32, (label, rel)


def _run(x, W, b, dev, expanded=False):
    h = eq.prepare_weights(W.to(dev), expanded=expanded)
    xd, bd = x.to(dev), (None if b is None else b.to(dev))
    y = eq.forward_expanded(h, xd, bd) if expanded else eq.forward(h, xd, bd)
    torch.cuda.synchronize()
    return h, y


@pytest.mark.parametrize("expanded", [False, True], ids=["spectral", "expanded"])
@pytest.mark.parametrize("w", WORKLOADS, ids=[w.name for w in WORKLOADS])
def test_workload_ragged_full_compare(w, expanded, cuda_device):
    N = w.N if w.N <= 64 else 517
    x, W, b = make_inputs(w.G, w.C_in, w.C_out, N, w.dtype, seed=0)
    h, y = _run(x, W, b, cuda_device, expanded)
    print(f"[kernel] {h.describe()}", flush=True)
    _check(y, oracle.forward(x, W, b), w.dtype, f"{w.name} N={N} {'expanded' if expanded else 'spectral'}")


@pytest.mark.parametrize("w", WORKLOADS, ids=[w.name for w in WORKLOADS])
def test_workload_full_size_all_tokens(w, cuda_device):
    # every token of the full workload, spectral and expanded, in the launch configuration the
    # benchmark times (same N, so the same grid, tile rounds and XCD grouping), against one oracle pass
    x, W, b = make_inputs(w.G, w.C_in, w.C_out, w.N, w.dtype, seed=0)
    h = eq.prepare_weights(W.to(cuda_device), expanded=True)
    xd, bd = x.to(cuda_device), b.to(cuda_device)
    outs = {"spectral": eq.forward(h, xd, bd), "expanded": eq.forward_expanded(h, xd, bd)}
    torch.cuda.synchronize()
    print(f"[kernel] {h.describe()}", flush=True)
    errs = compare_all_tokens(outs, lambda lo, hi: oracle.forward(x[lo:hi], W, b), w.N, chunk=2048)
    for k, e in errs.items():
        print(f"[parity] {w.name} full N={w.N} all tokens {k}: rel_frob={e.rel:.3e} max_abs={e.max_abs:.3e}",
              flush=True)
        assert e.finite, (w.name, k)
        if w.dtype == "bf16":
            assert e.rel <= REL_BF16 and e.max_abs <= MAX_BF16, (w.name, k, e.rel, e.max_abs)
        else:
            assert e.rel <= REL_F32, (w.name, k, e.rel)


# Wide outputs make many output tiles, so on a 256-CU device each persistent workgroup of the
# large-channel kernel walks several token tiles at small N: this exercises the hand-over between
# tiles (the load pipeline crossing tile boundaries, a tile's outputs stored during the next tile's
# stages, the last tile's own flush) including a ragged last tile and rows that are not a whole
# number of 16-byte pieces (C_out * G not a multiple of 8). C_in = 200 pads the channel stages: the
# last stage's loads past C_in re-read real channels, which meet zero weight columns.
@pytest.mark.parametrize("with_bias", [True, False], ids=["bias", "nobias"])
@pytest.mark.parametrize("expanded", [False, True], ids=["spectral", "expanded"])
@pytest.mark.parametrize("G,C_in,C_out", [(4, 128, 4096), (8, 64, 2048), (4, 128, 4095), (2, 128, 4096),
                                          (1, 256, 4096), (8, 200, 1024), (4, 200, 2048), (4, 384, 4095),
                                          (8, 320, 1024)])
def test_large_channel_multi_tile(G, C_in, C_out, expanded, with_bias, cuda_device):
    if expanded and G == 1:
        pytest.skip("G = 1 has no separate expanded form")
    if not with_bias and G in (2, 1):
        pytest.skip("the no-bias case is covered at G = 4 and 8")
    N = 3001
    x, W, b = make_inputs(G, C_in, C_out, N, "bf16", seed=3)
    if not with_bias:
        b = None
    h, y = _run(x, W, b, cuda_device, expanded)
    desc = h.describe()
    print(f"[kernel] {desc}", flush=True)
    # (G = 4 and 8 with C_in up to 256: the resident-planes kernels, which keep a token tile's planes on chip)
    kern = desc.split("|")[2 if expanded else 1]
    assert "big" in kern or (G in (4, 8) and C_in <= 256 and not expanded and "resident" in kern), desc
    _check(y, oracle.forward(x, W, b), "bf16",
           f"G={G} {C_in}->{C_out} N={N} {'expanded' if expanded else 'spectral'} all tokens")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("N", [1, 17, 1000])
def test_edge_token_counts_and_groups(G, N, dtype, cuda_device):
    C_in, C_out = 32, 48
    x, W, b = make_inputs(G, C_in, C_out, N, dtype, seed=G * 1000 + N)
    for bias in (b, None):
        for expanded in (False, True):
            _, y = _run(x, W, bias, cuda_device, expanded)
            _check(y, oracle.forward(x, W, bias), dtype,
                   f"G={G} N={N} {dtype} bias={bias is not None} expanded={expanded}")


@pytest.mark.parametrize("dtype,C_in,C_out", [("bf16", 40, 20), ("bf16", 8, 1), ("bf16", 136, 200),
                                              ("bf16", 96, 200), ("bf16", 96, 100), ("bf16", 64, 54),
                                              ("f32", 5, 3), ("f32", 70, 130)])
@pytest.mark.parametrize("G", [4, 8])
def test_ragged_channels(G, dtype, C_in, C_out, cuda_device):
    N = 203
    x, W, b = make_inputs(G, C_in, C_out, N, dtype, seed=7)
    for expanded in (False, True):
        _, y = _run(x, W, b, cuda_device, expanded)
        _check(y, oracle.forward(x, W, b), dtype, f"G={G} C_in={C_in} C_out={C_out} {dtype} exp={expanded}")


def test_empty_batch(cuda_device):
    x, W, b = make_inputs(4, 32, 32, 0, "bf16")
    h, y = _run(x, W, b, cuda_device, expanded=True)
    assert y.shape == (0, 32, 4)
    y2 = eq.forward_expanded(h, x.to(cuda_device), b.to(cuda_device))
    assert y2.shape == (0, 32, 4)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_spectral_weights_match_oracle_dft(G, dtype, cuda_device):
    C_out, C_in = 40, 48
    _, W, _ = make_inputs(G, C_in, C_out, 1, dtype, seed=3)
    h = eq.prepare_weights(W.to(cuda_device))
    got = eq.export_spectral_weights(h).cpu().double().numpy()
    Wh = oracle.dft_weights(W)  # [C_out, C_in, G/2+1] complex
    planes = [Wh[:, :, 0].real]
    if G >= 2:
        planes.append(Wh[:, :, G // 2].real)
    for k in range(1, G // 2):
        planes += [Wh[:, :, k].real, Wh[:, :, k].imag]
    ref = np.stack(planes)
    # The oracle's own fp64 error: its twiddles cos/sin(2 pi d k / G) are not exactly 0 at multiples
    # of pi/2, so an exactly-zero coefficient comes out near 1e-17 there; bound it by G eps sum|W|.
    floor = 4 * G * np.finfo(np.float64).eps * np.abs(W.double().numpy()).sum(axis=2)[None]
    if dtype == "bf16":
        # one bf16 rounding of an fp32 value: within half a bf16 ulp (2^-8 relative) of the exact DFT
        tol = np.abs(ref) * 2.0 ** -8 + floor
    else:
        tol = np.abs(ref) * 1e-6 + 1e-7
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (int(bad.sum()), got[bad][:5], ref[bad][:5])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_expanded_weight_is_exact_unrolling(G, dtype, cuda_device):
    _, W, _ = make_inputs(G, 16, 24, 1, dtype, seed=4)
    h = eq.prepare_weights(W.to(cuda_device), expanded=True)
    got = eq.export_expanded_weight(h).cpu().double().numpy()
    np.testing.assert_array_equal(got, oracle.expand(W))


@pytest.mark.parametrize("w", WORKLOADS[1:], ids=[w.name for w in WORKLOADS[1:]])
def test_equivariance_full_size(w, cuda_device):
    # cyclic shift of x along g shifts y along h (holds at any size), at every bf16 workload's full size
    # in the benchmark's launch configuration
    x, W, b = make_inputs(w.G, w.C_in, w.C_out, w.N, w.dtype, seed=0)
    h = eq.prepare_weights(W.to(cuda_device))
    xd, bd = x.to(cuda_device), b.to(cuda_device)
    y = eq.forward(h, xd, bd).double()
    for s in range(1, w.G):
        ys = eq.forward(h, torch.roll(xd, s, dims=2), bd).double()
        rel = (torch.linalg.vector_norm(ys - torch.roll(y, s, dims=2)) / torch.linalg.vector_norm(y)).item()
        print(f"[equivariance] shift={s} rel={rel:.3e}", flush=True)
        assert rel <= 1e-2


@pytest.mark.parametrize("w", WORKLOADS[1:], ids=[w.name for w in WORKLOADS[1:]])
def test_deterministic(w, cuda_device):
    x, W, b = make_inputs(w.G, w.C_in, w.C_out, 2048, w.dtype, seed=5)
    h = eq.prepare_weights(W.to(cuda_device), expanded=True)
    xd, bd = x.to(cuda_device), b.to(cuda_device)
    assert torch.equal(eq.forward(h, xd, bd), eq.forward(h, xd, bd))
    assert torch.equal(eq.forward_expanded(h, xd, bd), eq.forward_expanded(h, xd, bd))


def test_abi_rejects_bad_pointers_with_device_tensors(cuda_device):
    lib = eq.load_library()
    x, W, b = make_inputs(4, 32, 32, 64, "bf16")
    h = eq.prepare_weights(W.to(cuda_device), expanded=True)
    xd = x.to(cuda_device)
    y = torch.empty((64, 32, 4), dtype=torch.bfloat16, device=cuda_device)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hp = ctypes.c_void_p(h.ptr)
    mis = ctypes.c_void_p(xd.data_ptr() + 2)
    assert lib.eqlin_forward(hp, mis, None, ctypes.c_void_p(y.data_ptr()), 63, s) == eq.EQLIN_ERR_INVALID_ARG
    assert lib.eqlin_forward(hp, ctypes.c_void_p(xd.data_ptr()), None, None, 64, s) == eq.EQLIN_ERR_INVALID_ARG
    assert lib.eqlin_forward(hp, ctypes.c_void_p(xd.data_ptr()), None, ctypes.c_void_p(y.data_ptr()), -1, s) \
        == eq.EQLIN_ERR_INVALID_ARG
    # in-place (x and y overlap) is rejected
    assert lib.eqlin_forward(hp, ctypes.c_void_p(xd.data_ptr()), None, ctypes.c_void_p(xd.data_ptr()), 64, s) \
        == eq.EQLIN_ERR_INVALID_ARG
    h2 = eq.prepare_weights(W.to(cuda_device), expanded=False)
    assert lib.eqlin_forward_expanded(ctypes.c_void_p(h2.ptr), ctypes.c_void_p(xd.data_ptr()), None,
                                      ctypes.c_void_p(y.data_ptr()), 64, s) == eq.EQLIN_ERR_INVALID_ARG
    with pytest.raises(eq.EqlinError):
        eq.prepare_weights(torch.zeros((4, 12, 4), dtype=torch.bfloat16, device=cuda_device))


@pytest.mark.parametrize("wi,N", [(1, 4096), (2, 4096), (3, 9000), (4, 4096)],
                         ids=["p4_c96", "p8_c64", "p4_c192x768", "p8_c256x1024"])
def test_graph_replay_matches_eager(wi, N, cuda_device):
    # The benchmark times HIP-graph replays; every replay must equal the eager result, also with
    # other eager work and synchronisations between replays. One case per kernel the workloads run
    # (p4/192->768 above the batch-size switch, so the resident-planes kernel; p8/256->1024 the G = 8
    # resident kernel, whose range table is a by-value kernel argument captured with the graph).
    w = WORKLOADS[wi]
    x, W, b = make_inputs(w.G, w.C_in, w.C_out, N, w.dtype, seed=9)
    h = eq.prepare_weights(W.to(cuda_device), expanded=True)
    x0, x1, bd = x.to(cuda_device), (x.float() * 0.5).to(torch.bfloat16).to(cuda_device), b.to(cuda_device)
    ref0, ref1 = eq.forward(h, x0, bd), eq.forward_expanded(h, x1, bd)
    y0, y1 = torch.empty_like(ref0), torch.empty_like(ref1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        eq.forward(h, x0, bd, y0)
        eq.forward_expanded(h, x1, bd, y1)
    for r in range(4):
        y0.zero_()
        y1.fill_(float("nan"))
        eq.forward(h, x1, None)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y0, ref0) and torch.equal(y1, ref1), f"replay {r}"


def test_lds_limit_refusal_falls_back_to_large_channel_kernel(cuda_device):
    # A device that refuses the small-channel kernel's LDS request (simulated by the library's fault
    # injection, EQLIN_FAULT_LDS_LIMIT) gets the large-channel kernel at prepare, not an error at the
    # first forward. Run in a child process: the setting is read when the library sizes LDS.
    import os
    import subprocess
    import sys

    code = (
        "import numpy as np, torch, fourier_domain_linear_amd as eq, oracle\n"
        "from fourier_domain_linear_amd.workloads import make_inputs\n"
        "x, W, b = make_inputs(4, 96, 96, 777, 'bf16', seed=2)\n"
        "h = eq.prepare_weights(W.cuda())\n"
        "y = eq.forward(h, x.cuda(), b.cuda()); torch.cuda.synchronize()\n"
        "ref = oracle.forward(x, W, b); d = y.double().cpu().numpy() - ref\n"
        "rel = np.linalg.norm(d) / np.linalg.norm(ref); mx = np.abs(d).max()\n"
        "print('DESC', h.describe()); print('ERR', rel, mx)\n"
        "assert rel <= 1e-2 and mx <= 3e-2\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, EQLIN_FAULT_LDS_LIMIT="65536", PYTHONPATH=root)
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True, text=True, timeout=300)
    print(r.stdout, r.stderr[-2000:], flush=True)
    assert r.returncode == 0, r.stderr[-2000:]
    desc = [l for l in r.stdout.splitlines() if l.startswith("DESC")][0]
    assert "forward: bf16 big" in desc, desc
