"""The C-ABI library loads and exports every symbol include/eqlin.h declares; host-side argument
checks return status codes without touching a GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import fourier_domain_linear_amd as eq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "eqlin.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(eqlin_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(eq.LIB_PATH):
        pytest.fail("libeqlin.so is not built: run `python -m fourier_domain_linear_amd.build`")
    return eq.load_library()


def test_header_declares_what_binding_lists():
    assert _declared() == sorted(eq.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert re.fullmatch(r"\d+\.\d+\.\d+", eq.version())
    assert eq.status_string(0) == "EQLIN_OK"
    assert eq.status_string(2) == "EQLIN_ERR_UNSUPPORTED"
    assert eq.status_string(99) == "EQLIN_ERR_UNKNOWN"


def _prepare(lib, W, C_out, C_in, G, dtype=1, flags=0, out=True):
    h = ctypes.c_void_p()
    return lib.eqlin_prepare_weights(W, C_out, C_in, G, dtype, flags, None, ctypes.byref(h) if out else None), h


def test_prepare_argument_errors(lib):
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every case fails its host-side check first
    assert _prepare(lib, fake, 4, 8, 4, out=False)[0] == eq.EQLIN_ERR_INVALID_ARG
    st, h = _prepare(lib, None, 4, 8, 4)
    assert st == eq.EQLIN_ERR_INVALID_ARG and h.value is None
    assert _prepare(lib, fake, 4, 8, 3)[0] == eq.EQLIN_ERR_INVALID_ARG         # G not a valid group
    assert _prepare(lib, fake, 4, 8, 16)[0] == eq.EQLIN_ERR_INVALID_ARG
    assert _prepare(lib, fake, 0, 8, 4)[0] == eq.EQLIN_ERR_INVALID_ARG         # C_out < 1
    assert _prepare(lib, fake, 4, -1, 4)[0] == eq.EQLIN_ERR_INVALID_ARG
    assert _prepare(lib, fake, 4, 8, 4, dtype=7)[0] == eq.EQLIN_ERR_INVALID_ARG
    assert _prepare(lib, fake, 4, 12, 4, dtype=eq.EQLIN_F16)[0] == eq.EQLIN_ERR_UNSUPPORTED  # f16, C_in % 8
    assert _prepare(lib, fake, 4, 8, 4, flags=0x10)[0] == eq.EQLIN_ERR_INVALID_ARG
    # the known flags together pass the flag check (and fail on the next one, the bf16 C_in rule)
    allf = eq.EQLIN_PREPARE_EXPANDED | eq.EQLIN_PREPARE_BACKWARD | eq.EQLIN_PREPARE_FIXED_KERNEL
    assert _prepare(lib, fake, 8, 12, 4, dtype=1, flags=allf)[0] == eq.EQLIN_ERR_UNSUPPORTED
    assert "C_in" in lib.eqlin_last_error().decode()
    assert _prepare(lib, ctypes.c_void_p(0x10008), 4, 8, 4)[0] == eq.EQLIN_ERR_INVALID_ARG  # misaligned
    assert _prepare(lib, fake, 4, 12, 4, dtype=1)[0] == eq.EQLIN_ERR_UNSUPPORTED  # bf16, C_in % 8
    assert "C_in" in lib.eqlin_last_error().decode()
    # the backward weights need C_out % 8 == 0 in bf16 (C_out is their C_in)
    assert _prepare(lib, fake, 12, 8, 4, dtype=1, flags=eq.EQLIN_PREPARE_BACKWARD)[0] == eq.EQLIN_ERR_UNSUPPORTED
    assert "C_out" in lib.eqlin_last_error().decode()
    assert _prepare(lib, fake, 4, 8, 4, flags=eq.EQLIN_PREPARE_D4)[0] == eq.EQLIN_ERR_INVALID_ARG  # D4 needs G = 8
    assert "D4" in lib.eqlin_last_error().decode()
    assert _prepare(lib, fake, (1 << 18) + 1, 8, 4)[0] == eq.EQLIN_ERR_UNSUPPORTED  # C_out * G > 2^20
    assert _prepare(lib, fake, 8, (1 << 17) + 8, 8)[0] == eq.EQLIN_ERR_UNSUPPORTED  # C_in * G > 2^20
    assert "2^20" in lib.eqlin_last_error().decode()


def test_forward_null_handle(lib):
    assert lib.eqlin_forward(None, None, None, None, 10, None) == eq.EQLIN_ERR_INVALID_ARG
    assert lib.eqlin_forward_expanded(None, None, None, None, 10, None) == eq.EQLIN_ERR_INVALID_ARG
    assert lib.eqlin_forward_act(None, None, None, None, 10, eq.EQLIN_ACT_GELU, None) == eq.EQLIN_ERR_INVALID_ARG
    assert lib.eqlin_forward_expanded_act(None, None, None, None, 10, eq.EQLIN_ACT_GELU, None) == \
        eq.EQLIN_ERR_INVALID_ARG
    assert lib.eqlin_destroy(None) == eq.EQLIN_OK
    assert lib.eqlin_export_spectral_weights(None, None, None) == eq.EQLIN_ERR_INVALID_ARG
    n = lib.eqlin_describe(None, None, 0)
    assert n > 0


def test_backward_null_handle(lib):
    assert lib.eqlin_backward_data(None, None, None, 10, None) == eq.EQLIN_ERR_INVALID_ARG
    assert lib.eqlin_backward_weights(None, None, None, None, None, 10, None, 0, None) == eq.EQLIN_ERR_INVALID_ARG
    assert lib.eqlin_backward_weights_workspace(None, 10) == 0
