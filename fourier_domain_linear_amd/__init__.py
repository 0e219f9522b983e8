"""MI355X-native EQ-Linear forward: a thin ctypes binding over libeqlin.so (include/eqlin.h).

The binding only marshals arguments (shape/dtype/device checks, pointers, the current HIP stream);
every step of the layer runs in the library's HIP kernels. There is no CPU fallback: if the library
is missing, every call raises.

    import fourier_domain_linear_amd as eq
    h = eq.prepare_weights(W)                 # W: cuda tensor [C_out, C_in, G], bf16 or fp32
    y = eq.forward(h, x, b)                   # x: [N, C_in, G]; b: [C_out] or None
    y2 = eq.forward_expanded(h, x, b)         # needs prepare_weights(W, expanded=True)
    dx = eq.backward_data(h, dy)              # needs prepare_weights(W, backward=True)
    dW, db = eq.backward_weights(h, x, dy)    # float32 gradients of W and b
    z = eq.forward(h, x, b, act="gelu")       # GELU(y), applied in the kernel's epilogue
    y = eq.mlp_block(h1, b1, h2, b2, x)       # EQ-Linear(C -> 4C), GELU, EQ-Linear(4C -> C)
    hc = eq.prepare_conv_weights(psi)         # p4 group convolution, psi [C_out, C_in, 4, k, k]
    y = eq.conv_forward(hc, x, b)             # x [B, H, W, C_in, 4] -> y [B, H, W, C_out, 4]

Method: "Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise Discrete Fourier
Transform" (explainer page, gist.science/es/paper/2607.21271).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libeqlin.so")

EQLIN_OK = 0
EQLIN_ERR_INVALID_ARG = 1
EQLIN_ERR_UNSUPPORTED = 2
EQLIN_ERR_OUT_OF_MEMORY = 3
EQLIN_ERR_HIP = 4
EQLIN_F32 = 0
EQLIN_BF16 = 1
EQLIN_F16 = 2
EQLIN_PREPARE_EXPANDED = 1
EQLIN_PREPARE_BACKWARD = 2
EQLIN_PREPARE_D4 = 4
EQLIN_PREPARE_FIXED_KERNEL = 8
GROUPS = ("cyclic", "d4")
EQLIN_ACT_NONE = 0
EQLIN_ACT_GELU = 1
_ACTS = {None: EQLIN_ACT_NONE, "none": EQLIN_ACT_NONE, "gelu": EQLIN_ACT_GELU}

# Every symbol include/eqlin.h declares.
EXPORTED = (
    "eqlin_prepare_weights", "eqlin_forward", "eqlin_forward_expanded", "eqlin_forward_act",
    "eqlin_forward_expanded_act", "eqlin_backward_data", "eqlin_backward_data_expanded",
    "eqlin_backward_weights_workspace", "eqlin_backward_weights", "eqlin_backward_weights_static", "eqlin_destroy",
    "eqlin_export_spectral_weights", "eqlin_export_expanded_weight", "eqlin_describe",
    "eqlin_status_string", "eqlin_last_error", "eqlin_version",
    "eqlin_prepare_conv_weights", "eqlin_conv_forward", "eqlin_conv_forward_expanded",
)

_lib = None


class EqlinError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load libeqlin.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m fourier_domain_linear_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint
    lib.eqlin_prepare_weights.argtypes = [vp, i32, i32, i32, i32, u32, vp, ctypes.POINTER(vp)]
    lib.eqlin_forward.argtypes = [vp, vp, vp, vp, i64, vp]
    lib.eqlin_forward_expanded.argtypes = [vp, vp, vp, vp, i64, vp]
    lib.eqlin_forward_act.argtypes = [vp, vp, vp, vp, i64, i32, vp]
    lib.eqlin_forward_expanded_act.argtypes = [vp, vp, vp, vp, i64, i32, vp]
    lib.eqlin_backward_data.argtypes = [vp, vp, vp, i64, vp]
    lib.eqlin_backward_data_expanded.argtypes = [vp, vp, vp, i64, vp]
    lib.eqlin_backward_weights_workspace.argtypes = [vp, i64]
    lib.eqlin_backward_weights_workspace.restype = ctypes.c_size_t
    lib.eqlin_backward_weights.argtypes = [vp, vp, vp, vp, vp, i64, vp, ctypes.c_size_t, vp]
    lib.eqlin_backward_weights_static.argtypes = [vp, vp, vp, vp, vp, i64, vp]
    lib.eqlin_prepare_conv_weights.argtypes = [vp, i32, i32, i32, i32, i32, u32, vp, ctypes.POINTER(vp)]
    lib.eqlin_conv_forward.argtypes = [vp, vp, vp, vp, i64, i32, i32, vp]
    lib.eqlin_conv_forward_expanded.argtypes = [vp, vp, vp, vp, i64, i32, i32, vp]
    lib.eqlin_destroy.argtypes = [vp]
    lib.eqlin_export_spectral_weights.argtypes = [vp, vp, vp]
    lib.eqlin_export_expanded_weight.argtypes = [vp, vp, vp]
    lib.eqlin_describe.argtypes = [vp, ctypes.c_char_p, ctypes.c_size_t]
    lib.eqlin_describe.restype = i32
    lib.eqlin_status_string.argtypes = [i32]
    lib.eqlin_status_string.restype = ctypes.c_char_p
    lib.eqlin_last_error.argtypes = []
    lib.eqlin_last_error.restype = ctypes.c_char_p
    lib.eqlin_version.argtypes = []
    lib.eqlin_version.restype = ctypes.c_char_p
    for name in ("eqlin_prepare_weights", "eqlin_forward", "eqlin_forward_expanded", "eqlin_destroy",
                 "eqlin_forward_act", "eqlin_forward_expanded_act", "eqlin_backward_data", "eqlin_backward_weights",
                 "eqlin_backward_data_expanded",
                 "eqlin_backward_weights_static", "eqlin_prepare_conv_weights", "eqlin_conv_forward",
                 "eqlin_conv_forward_expanded",
                 "eqlin_export_spectral_weights", "eqlin_export_expanded_weight"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != EQLIN_OK:
        lib = load_library()
        name = lib.eqlin_status_string(status).decode()
        detail = lib.eqlin_last_error().decode()
        raise EqlinError(status, f"{what}: {name}: {detail}")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return EQLIN_BF16
    if dt == torch.float16:
        return EQLIN_F16
    if dt == torch.float32:
        return EQLIN_F32
    raise TypeError(f"unsupported dtype {dt} (bfloat16, float16 or float32)")


def _need_cuda(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Handle:
    """Owns an eqlin_handle_t; destroyed with the object (or explicitly via destroy())."""

    def __init__(self, ptr: int, C_out: int, C_in: int, G: int, dtype: torch.dtype, device, expanded: bool,
                 backward: bool = False, group: str = "cyclic", conv_k: int = 0):
        self.ptr = ptr
        self.conv_k = conv_k
        self.C_out, self.C_in, self.G, self.group = C_out, C_in, G, group
        self.dtype, self.device, self.expanded, self.backward = dtype, device, expanded, backward

    def destroy(self):
        if self.ptr:
            load_library().eqlin_destroy(ctypes.c_void_p(self.ptr))
            self.ptr = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    def describe(self) -> str:
        return describe(self)


def prepare_weights(W: torch.Tensor, expanded: bool = False, backward: bool = False, group: str = "cyclic",
                    fixed_kernel: bool = False) -> Handle:
    """eqlin_prepare_weights: W [C_out, C_in, G] (cuda, bf16 or fp32) -> Handle. ``expanded`` builds the
    unrolled comparator, ``backward`` the weights of backward_data. ``group``: "cyclic" (G = 1, 2, 4, 8)
    or "d4", the dihedral group of the square (G = 8, element a + 4b = r^a s^b; EQLIN_PREPARE_D4).
    ``fixed_kernel``: one forward kernel for every batch size (EQLIN_PREPARE_FIXED_KERNEL)."""
    if group not in GROUPS:
        raise ValueError(f"group must be one of {GROUPS}, got {group!r}")
    lib = load_library()
    _need_cuda(W, "W")
    if W.dim() != 3:
        raise ValueError(f"W must be [C_out, C_in, G], got {tuple(W.shape)}")
    C_out, C_in, G = W.shape
    out = ctypes.c_void_p()
    flags = (EQLIN_PREPARE_EXPANDED if expanded else 0) | (EQLIN_PREPARE_BACKWARD if backward else 0) | \
        (EQLIN_PREPARE_D4 if group == "d4" else 0) | (EQLIN_PREPARE_FIXED_KERNEL if fixed_kernel else 0)
    with torch.cuda.device(W.device):
        st = lib.eqlin_prepare_weights(ctypes.c_void_p(W.data_ptr()), C_out, C_in, G, _dtype_code(W.dtype),
                                       flags, _stream(W), ctypes.byref(out))
    _check(st, "eqlin_prepare_weights")
    return Handle(out.value, C_out, C_in, G, W.dtype, W.device, expanded, backward, group)


def _act_code(act) -> int:
    if act not in _ACTS:
        raise ValueError(f"act must be one of {sorted(k for k in _ACTS if k)} or None, got {act!r}")
    return _ACTS[act]


def _forward(fn, what: str, h: Handle, x: torch.Tensor, b: torch.Tensor | None, y: torch.Tensor | None,
             act: int | None = None):
    _need_cuda(x, "x")
    if x.dtype != h.dtype:
        raise TypeError(f"x dtype {x.dtype} != handle dtype {h.dtype}")
    if x.dim() != 3 or x.shape[1] != h.C_in or x.shape[2] != h.G:
        raise ValueError(f"x must be [N, {h.C_in}, {h.G}], got {tuple(x.shape)}")
    N = x.shape[0]
    if y is None:
        y = torch.empty((N, h.C_out, h.G), dtype=x.dtype, device=x.device)
    else:
        _need_cuda(y, "y")
        if y.dtype != h.dtype or tuple(y.shape) != (N, h.C_out, h.G):
            raise ValueError(f"y must be [{N}, {h.C_out}, {h.G}] of {h.dtype}")
    bp = None
    if b is not None:
        _need_cuda(b, "b")
        if b.dtype != h.dtype or tuple(b.shape) != (h.C_out,):
            raise ValueError(f"b must be [{h.C_out}] of {h.dtype}")
        bp = ctypes.c_void_p(b.data_ptr())
    args = (ctypes.c_void_p(h.ptr), ctypes.c_void_p(x.data_ptr()), bp, ctypes.c_void_p(y.data_ptr()), N)
    with torch.cuda.device(x.device):
        st = fn(*args, _stream(x)) if act is None else fn(*args, act, _stream(x))
    _check(st, what)
    return y


def forward(h: Handle, x: torch.Tensor, b: torch.Tensor | None = None, y: torch.Tensor | None = None,
            act: str | None = None):
    """eqlin_forward: y[n, o, h] = b[o] + sum_{i,g} W[o, i, (h-g) mod G] x[n, i, g] (spectral kernel).
    act="gelu" calls eqlin_forward_act instead, which applies GELU to y in the kernel's epilogue."""
    lib = load_library()
    if _act_code(act) == EQLIN_ACT_NONE:
        return _forward(lib.eqlin_forward, "eqlin_forward", h, x, b, y)
    return _forward(lib.eqlin_forward_act, "eqlin_forward_act", h, x, b, y, _act_code(act))


def forward_expanded(h: Handle, x: torch.Tensor, b: torch.Tensor | None = None, y: torch.Tensor | None = None,
                     act: str | None = None):
    """eqlin_forward_expanded: the same layer as one dense product with the unrolled weight (with
    act="gelu": eqlin_forward_expanded_act)."""
    if not h.expanded:
        raise ValueError("handle was prepared without expanded=True")
    lib = load_library()
    if _act_code(act) == EQLIN_ACT_NONE:
        return _forward(lib.eqlin_forward_expanded, "eqlin_forward_expanded", h, x, b, y)
    return _forward(lib.eqlin_forward_expanded_act, "eqlin_forward_expanded_act", h, x, b, y, _act_code(act))


def mlp_block(h1: Handle, b1: torch.Tensor | None, h2: Handle, b2: torch.Tensor | None, x: torch.Tensor,
              hidden: torch.Tensor | None = None, y: torch.Tensor | None = None, expanded: bool = False):
    """The transformer MLP block as two library calls on the current stream: hidden = GELU(layer 1 (x))
    with GELU in layer 1's epilogue, then y = layer 2 (hidden). h1: [C_h, C, G] weights, h2: [C, C_h, G].
    expanded=True runs both layers as dense products with the unrolled weights (the comparator)."""
    if h1.C_out != h2.C_in or h1.G != h2.G or h1.dtype != h2.dtype or h1.group != h2.group:
        raise ValueError("layer 2 must take layer 1's outputs (C_in, G and dtype)")
    fwd = forward_expanded if expanded else forward
    hidden = fwd(h1, x, b1, hidden, act="gelu")
    return fwd(h2, hidden, b2, y)


def backward_data(h: Handle, dy: torch.Tensor, dx: torch.Tensor | None = None) -> torch.Tensor:
    """eqlin_backward_data: dx[n, i, g] = sum_{o, h} W[o, i, (h-g) mod G] dy[n, o, h]."""
    if not h.backward:
        raise ValueError("handle was prepared without backward=True")
    _need_cuda(dy, "dy")
    if dy.dtype != h.dtype or dy.dim() != 3 or dy.shape[1] != h.C_out or dy.shape[2] != h.G:
        raise ValueError(f"dy must be [N, {h.C_out}, {h.G}] of {h.dtype}, got {tuple(dy.shape)} {dy.dtype}")
    N = dy.shape[0]
    if dx is None:
        dx = torch.empty((N, h.C_in, h.G), dtype=dy.dtype, device=dy.device)
    else:
        _need_cuda(dx, "dx")
        if dx.dtype != h.dtype or tuple(dx.shape) != (N, h.C_in, h.G):
            raise ValueError(f"dx must be [{N}, {h.C_in}, {h.G}] of {h.dtype}")
    with torch.cuda.device(dy.device):
        st = load_library().eqlin_backward_data(ctypes.c_void_p(h.ptr), ctypes.c_void_p(dy.data_ptr()),
                                                ctypes.c_void_p(dx.data_ptr()), N, _stream(dy))
    _check(st, "eqlin_backward_data")
    return dx


def backward_data_expanded(h: Handle, dy: torch.Tensor, dx: torch.Tensor | None = None) -> torch.Tensor:
    """eqlin_backward_data_expanded: the same dx as one dense product with the unrolled weight (needs
    prepare_weights(W, expanded=True, backward=True))."""
    if not (h.backward and h.expanded):
        raise ValueError("handle was prepared without expanded=True and backward=True")
    _need_cuda(dy, "dy")
    if dy.dtype != h.dtype or dy.dim() != 3 or dy.shape[1] != h.C_out or dy.shape[2] != h.G:
        raise ValueError(f"dy must be [N, {h.C_out}, {h.G}] of {h.dtype}, got {tuple(dy.shape)} {dy.dtype}")
    N = dy.shape[0]
    if dx is None:
        dx = torch.empty((N, h.C_in, h.G), dtype=dy.dtype, device=dy.device)
    else:
        _need_cuda(dx, "dx")
        if dx.dtype != h.dtype or tuple(dx.shape) != (N, h.C_in, h.G):
            raise ValueError(f"dx must be [{N}, {h.C_in}, {h.G}] of {h.dtype}")
    with torch.cuda.device(dy.device):
        st = load_library().eqlin_backward_data_expanded(ctypes.c_void_p(h.ptr), ctypes.c_void_p(dy.data_ptr()),
                                                         ctypes.c_void_p(dx.data_ptr()), N, _stream(dy))
    _check(st, "eqlin_backward_data_expanded")
    return dx


def backward_weights_workspace(h: Handle, N: int) -> int:
    """Bytes of device scratch eqlin_backward_weights needs for N tokens."""
    return int(load_library().eqlin_backward_weights_workspace(ctypes.c_void_p(h.ptr), int(N)))


def backward_weights(h: Handle, x: torch.Tensor, dy: torch.Tensor, with_bias: bool = True,
                     workspace: torch.Tensor | None = None):
    """eqlin_backward_weights -> (dW float32 [C_out, C_in, G], db float32 [C_out] or None):
    dW[o, i, d] = sum_{n, h} dy[n, o, h] x[n, i, (h-d) mod G], db[o] = sum_{n, h} dy[n, o, h]."""
    _need_cuda(x, "x")
    _need_cuda(dy, "dy")
    if x.dtype != h.dtype or dy.dtype != h.dtype:
        raise TypeError(f"x and dy must be {h.dtype}")
    if x.dim() != 3 or x.shape[1:] != (h.C_in, h.G) or dy.dim() != 3 or dy.shape[1:] != (h.C_out, h.G) \
            or x.shape[0] != dy.shape[0]:
        raise ValueError(f"x must be [N, {h.C_in}, {h.G}] and dy [N, {h.C_out}, {h.G}]")
    N = x.shape[0]
    dW = torch.empty((h.C_out, h.C_in, h.G), dtype=torch.float32, device=x.device)
    db = torch.empty((h.C_out,), dtype=torch.float32, device=x.device) if with_bias else None
    need = backward_weights_workspace(h, N)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    wsp = ctypes.c_void_p(workspace.data_ptr()) if need else None
    with torch.cuda.device(x.device):
        st = load_library().eqlin_backward_weights(
            ctypes.c_void_p(h.ptr), ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(dy.data_ptr()),
            ctypes.c_void_p(dW.data_ptr()), ctypes.c_void_p(db.data_ptr()) if db is not None else None, N, wsp,
            need, _stream(x))
    _check(st, "eqlin_backward_weights")
    return dW, db


def prepare_conv_weights(psi: torch.Tensor, expanded: bool = False) -> Handle:
    """eqlin_prepare_conv_weights: psi [C_out, C_in, 4, k, k] (cuda, bf16 or fp16) -> Handle of the p4
    group convolution y[b, p, o, h] = bias[o] + sum psi[o, i, (h - g) mod 4, R^-h delta] x[b, p + delta, i, g].
    ``expanded`` also builds the unrolled comparator (conv_forward_expanded)."""
    lib = load_library()
    _need_cuda(psi, "psi")
    if psi.dim() != 5 or psi.shape[2] != 4 or psi.shape[3] != psi.shape[4]:
        raise ValueError(f"psi must be [C_out, C_in, 4, k, k], got {tuple(psi.shape)}")
    C_out, C_in, G, k, _ = psi.shape
    out = ctypes.c_void_p()
    with torch.cuda.device(psi.device):
        st = lib.eqlin_prepare_conv_weights(ctypes.c_void_p(psi.data_ptr()), C_out, C_in, G, k, _dtype_code(psi.dtype),
                                            EQLIN_PREPARE_EXPANDED if expanded else 0, _stream(psi), ctypes.byref(out))
    _check(st, "eqlin_prepare_conv_weights")
    return Handle(out.value, C_out, C_in, G, psi.dtype, psi.device, expanded, conv_k=k)


def _conv(fn, what: str, h: Handle, x: torch.Tensor, b: torch.Tensor | None, y: torch.Tensor | None):
    if not h.conv_k:
        raise ValueError("not a convolution handle (prepare_conv_weights)")
    _need_cuda(x, "x")
    if x.dtype != h.dtype or x.dim() != 5 or x.shape[3:] != (h.C_in, h.G):
        raise ValueError(f"x must be [B, H, W, {h.C_in}, {h.G}] of {h.dtype}, got {tuple(x.shape)} {x.dtype}")
    B, H, W = x.shape[:3]
    if y is None:
        y = torch.empty((B, H, W, h.C_out, h.G), dtype=x.dtype, device=x.device)
    else:
        _need_cuda(y, "y")
        if y.dtype != h.dtype or tuple(y.shape) != (B, H, W, h.C_out, h.G):
            raise ValueError(f"y must be [{B}, {H}, {W}, {h.C_out}, {h.G}] of {h.dtype}")
    bp = None
    if b is not None:
        _need_cuda(b, "b")
        if b.dtype != h.dtype or tuple(b.shape) != (h.C_out,):
            raise ValueError(f"b must be [{h.C_out}] of {h.dtype}")
        bp = ctypes.c_void_p(b.data_ptr())
    with torch.cuda.device(x.device):
        st = fn(ctypes.c_void_p(h.ptr), ctypes.c_void_p(x.data_ptr()), bp, ctypes.c_void_p(y.data_ptr()), B, H, W,
                _stream(x))
    _check(st, what)
    return y


def conv_forward(h: Handle, x: torch.Tensor, b: torch.Tensor | None = None, y: torch.Tensor | None = None):
    """eqlin_conv_forward: x [B, H, W, C_in, 4] -> y [B, H, W, C_out, 4] (the spectral kernel)."""
    return _conv(load_library().eqlin_conv_forward, "eqlin_conv_forward", h, x, b, y)


def conv_forward_expanded(h: Handle, x: torch.Tensor, b: torch.Tensor | None = None, y: torch.Tensor | None = None):
    """eqlin_conv_forward_expanded: the same through the unrolled gathered layer (needs expanded=True)."""
    if not h.expanded:
        raise ValueError("handle was prepared without expanded=True")
    return _conv(load_library().eqlin_conv_forward_expanded, "eqlin_conv_forward_expanded", h, x, b, y)


STATIC_SCRATCH_BYTES = 64 << 20  # EQLIN_STATIC_SCRATCH_BYTES


def backward_weights_static(h: Handle, x: torch.Tensor, dy: torch.Tensor, with_bias: bool = True):
    """eqlin_backward_weights_static: backward_weights with the library's static per-device scratch
    instead of a workspace (no device allocation in the library; the gradient tensors are allocated
    here unless passed in). Calls on one device must not overlap."""
    _need_cuda(x, "x")
    _need_cuda(dy, "dy")
    if x.dtype != h.dtype or dy.dtype != h.dtype:
        raise TypeError(f"x and dy must be {h.dtype}")
    if x.dim() != 3 or x.shape[1:] != (h.C_in, h.G) or dy.dim() != 3 or dy.shape[1:] != (h.C_out, h.G) \
            or x.shape[0] != dy.shape[0]:
        raise ValueError(f"x must be [N, {h.C_in}, {h.G}] and dy [N, {h.C_out}, {h.G}]")
    N = x.shape[0]
    dW = torch.empty((h.C_out, h.C_in, h.G), dtype=torch.float32, device=x.device)
    db = torch.empty((h.C_out,), dtype=torch.float32, device=x.device) if with_bias else None
    with torch.cuda.device(x.device):
        st = load_library().eqlin_backward_weights_static(
            ctypes.c_void_p(h.ptr), ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(dy.data_ptr()),
            ctypes.c_void_p(dW.data_ptr()), ctypes.c_void_p(db.data_ptr()) if db is not None else None, N,
            _stream(x))
    _check(st, "eqlin_backward_weights_static")
    return dW, db


def export_spectral_weights(h: Handle) -> torch.Tensor:
    """eqlin_export_spectral_weights -> float32 [G, C_out, C_in] (plane order in include/eqlin.h)."""
    out = torch.empty((h.G, h.C_out, h.C_in), dtype=torch.float32, device=h.device)
    with torch.cuda.device(h.device):
        st = load_library().eqlin_export_spectral_weights(ctypes.c_void_p(h.ptr), ctypes.c_void_p(out.data_ptr()),
                                                          _stream(out))
    _check(st, "eqlin_export_spectral_weights")
    return out


def export_expanded_weight(h: Handle) -> torch.Tensor:
    """eqlin_export_expanded_weight -> [C_out*G, C_in*G] of the handle's dtype."""
    out = torch.empty((h.C_out * h.G, h.C_in * h.G), dtype=h.dtype, device=h.device)
    with torch.cuda.device(h.device):
        st = load_library().eqlin_export_expanded_weight(ctypes.c_void_p(h.ptr), ctypes.c_void_p(out.data_ptr()),
                                                         _stream(out))
    _check(st, "eqlin_export_expanded_weight")
    return out


def describe(h: Handle) -> str:
    lib = load_library()
    buf = ctypes.create_string_buffer(512)
    lib.eqlin_describe(ctypes.c_void_p(h.ptr), buf, len(buf))
    return buf.value.decode()


def version() -> str:
    return load_library().eqlin_version().decode()


def status_string(code: int) -> str:
    return load_library().eqlin_status_string(code).decode()


def destroy(h: Handle):
    h.destroy()
