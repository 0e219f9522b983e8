"""Tensors at the size limits: the forward (and its unrolled comparator) on x and y of more than 2^31
bytes, for each kernel family -- the small-channel stream kernel, the resident-planes kernels at G = 4
and G = 8 (C_in <= 256), the large-channel G = 8 kernel (C_in > 256) and the large-channel kernel the
unrolled comparator runs on -- which address x and y with 64-bit bases per token tile (or row block)
and 32-bit offsets inside it, so no index may wrap past 2^31 bytes; and the convolution at the
largest batch its single 32-bit x range admits.

x is drawn on the device (torch's generator, seeded) to keep host memory small; the oracle sees the
same bf16 values of the sampled tokens, copied back: the first and last rows, the rows around the
2^31-byte points of x and of y, and random rows. Bars: the layer's (bf16: relative Frobenius error
<= 1e-2 and max abs error <= 3e-2).
"""
import numpy as np
import pytest
import torch

import fourier_domain_linear_amd as eq
import oracle
from fourier_domain_linear_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu

REL_BF16, MAX_BF16 = 1e-2, 3e-2


def _sample_rows(N, C_in, C_out, G, rng):
    rows = set(range(64)) | set(range(N - 64, N))
    for row_bytes in (C_in * G * 2, C_out * G * 2):
        edge = (1 << 31) // row_bytes
        rows |= set(range(max(0, edge - 32), min(N, edge + 32)))
    rows |= set(int(v) for v in rng.integers(0, N, 128))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("G,C_in,C_out,N,expanded,kernel", [
    (4, 16, 16, 1 << 25, True, "stream"),             # x and y 4.3 GB each
    (4, 256, 256, 1_200_000, True, "resident-planes"),  # (unrolled: the large-channel kernel at G = 1) 2.46 GB each
    (8, 256, 256, 640_000, False, "resident-planes"),   # 2.6 GB each
    (8, 512, 512, 300_000, False, "big"),               # 2.46 GB each
], ids=["stream_p4_c16_n33554432", "res_p4_c256_n1200000", "res8_p8_c256_n640000", "big_p8_c512_n300000"])
def test_forward_beyond_2gib(G, C_in, C_out, N, expanded, kernel, cuda_device):
    assert N * C_in * G * 2 > 1 << 31 and N * C_out * G * 2 > 1 << 31
    _, W, b = make_inputs(G, C_in, C_out, 1, "bf16", seed=3)
    gen = torch.Generator(device=cuda_device).manual_seed(17)
    x = torch.randn((N, C_in, G), generator=gen, device=cuda_device).to(torch.bfloat16)
    h = eq.prepare_weights(W.to(cuda_device), expanded=expanded)
    print(f"[case] G={G} {C_in}->{C_out} N={N} [{h.describe()}]", flush=True)
    assert f"forward: bf16 {kernel} " in h.describe(), h.describe()  # the kernel family this case is for
    bd = b.to(cuda_device)
    outs = {"spectral": eq.forward(h, x, bd)}
    if expanded:
        outs["expanded"] = eq.forward_expanded(h, x, bd)
    torch.cuda.synchronize()
    rows = _sample_rows(N, C_in, C_out, G, np.random.default_rng(5))
    idx = torch.from_numpy(rows).to(cuda_device)
    ref = oracle.forward(x.index_select(0, idx).cpu(), W, b)
    for name, y in outs.items():
        yv = y.index_select(0, idx).to("cpu", torch.float64).numpy()
        assert np.all(np.isfinite(yv)), name
        d = yv - ref
        rel = float(np.linalg.norm(d) / np.linalg.norm(ref))
        mx = float(np.max(np.abs(d)))
        print(f"[parity] G={G} {C_in}->{C_out} N={N} {name}, {len(rows)} rows: rel_frob={rel:.3e} max_abs={mx:.3e}",
              flush=True)
        assert rel <= REL_BF16 and mx <= MAX_BF16, (name, rel, mx)
    del outs, x
    torch.cuda.empty_cache()


def test_conv_at_the_x_limit(cuda_device):
    # the convolution addresses x with one 32-bit range: B*H*W*C_in*8 bytes must stay below 2^31. Here
    # 15 images of 256 x 256 pixels at C_in = 256: 2.01e9 bytes, the largest batch of such images. Each
    # sampled pixel's output is the oracle's on the k x k crop around it (zero-filled outside the
    # image, which is the convolution's zero padding).
    from oracle import conv
    from fourier_domain_linear_amd.workloads import make_conv_inputs

    B, H, W, C_in, C_out, k = 15, 256, 256, 256, 64, 3
    assert B * H * W * C_in * 8 < 1 << 31 and (B + 1) * H * W * C_in * 8 >= 1 << 31
    _, psi, b = make_conv_inputs(C_in, C_out, k, 1, 1, 1, "bf16", seed=9)
    gen = torch.Generator(device=cuda_device).manual_seed(23)
    x = torch.randn((B, H, W, C_in, 4), generator=gen, device=cuda_device).to(torch.bfloat16)
    h = eq.prepare_conv_weights(psi.to(cuda_device))
    print(f"[case] conv {B}x{H}x{W} {C_in}->{C_out} k={k} [{h.describe()}]", flush=True)
    y = eq.conv_forward(h, x, b.to(cuda_device))
    torch.cuda.synchronize()
    r = k // 2
    rng = np.random.default_rng(8)
    pix = [(0, 0, 0), (B - 1, H - 1, W - 1), (B - 1, 0, W - 1), (B - 1, H - 1, 0), (7, 128, 1)]
    pix += [(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(W))) for _ in range(27)]
    got, ref = [], []
    for (n, py, px) in pix:
        crop = torch.zeros((1, k, k, C_in, 4), dtype=torch.bfloat16)
        y0, y1, x0, x1 = max(0, py - r), min(H, py + r + 1), max(0, px - r), min(W, px + r + 1)
        crop[0, y0 - (py - r):y1 - (py - r), x0 - (px - r):x1 - (px - r)] = x[n, y0:y1, x0:x1].cpu()
        ref.append(conv.forward(crop, psi, b)[0, r, r])
        got.append(y[n, py, px].to("cpu", torch.float64).numpy())
    got, ref = np.stack(got), np.stack(ref)
    d = got - ref
    rel = float(np.linalg.norm(d) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(d)))
    print(f"[parity] conv at the x limit, {len(pix)} pixels: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert np.all(np.isfinite(got)) and rel <= REL_BF16 and mx <= MAX_BF16, (rel, mx)
    del x, y
    torch.cuda.empty_cache()
