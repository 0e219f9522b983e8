"""The oracle's pins must catch plausible mistakes: each case below plants one slip in a copy of
oracle/eqlin_oracle.c (a wrong index, a sign, a dropped term or bias), builds it, and runs
tests/test_oracle.py against that build in a child process, which must then fail. An unmodified
copy built the same way must pass, so a failure is the pins' doing and not the harness's. Every
slip keeps all memory accesses in bounds. The Python parts of the oracle (the D4 group and its
layer, the GELU and the MLP block, the p4 group convolution) get the same treatment through a copy of the oracle package
that the child process imports instead of the real one."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "eqlin_oracle.c")

MUTANTS = {
    # the unrolled weight read as a correlation, W[o, i, (g-h) mod G]
    "correlation_index": ("int64_t d = ((h - g) % G + G) % G;", "int64_t d = ((g - h) % G + G) % G;"),
    "bias_dropped": ("yn[r] = acc + (b ? b[r / G] : 0.0);", "yn[r] = acc;"),
    "bias_wrong_channel": ("yn[r] = acc + (b ? b[r / G] : 0.0);", "yn[r] = acc + (b ? b[r % C_out] : 0.0);"),
    "last_input_column_dropped": ("for (int64_t c = 0; c < cols; ++c) acc += er[c] * xn[c];",
                                  "for (int64_t c = 0; c + 1 < cols; ++c) acc += er[c] * xn[c];"),
    "dft_conjugated": ("si -= w * sin(ang);", "si += w * sin(ang);"),
    "dft_without_twiddle_product": ("(double)((d * k) % G)", "(double)((d + k) % G)"),
    "dx_last_output_row_dropped": ("for (int64_t r = 0; r < rows; ++r) acc += E[r * cols + c] * dyn[r];",
                                   "for (int64_t r = 0; r + 1 < rows; ++r) acc += E[r * cols + c] * dyn[r];"),
    "dw_folded_on_wrong_diagonal": ("acc += dE[h * cols + i * G + ((h - d) % G + G) % G];",
                                    "acc += dE[h * cols + i * G + ((h + d) % G + G) % G];"),
    "db_one_group_sample": ("bsum += d;", "bsum += (h == 0 ? d : 0.0);"),
    "dw_last_token_dropped": ("            for (int64_t h = 0; h < G; ++h) {\n                const double d = dy",
                              "            for (int64_t h = 0; h < G && n + 1 < N; ++h) {\n                const double d = dy"),
}


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    lib = tmp_path / f"{name}.so"
    src.write_text(text)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", str(src), "-o", str(lib), "-lm"],
                   check=True)
    return str(lib)


def _run_pins(lib):
    env = dict(os.environ, EQLIN_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"), "-x", "-q",
           "-p", "no:cacheprovider", "-m", "not gpu"]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def test_unmodified_copy_passes(tmp_path):
    r = _run_pins(_build(tmp_path, "same", open(SRC).read()))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"anchor for {name} not unique in eqlin_oracle.c"
    r = _run_pins(_build(tmp_path, name, text.replace(old, new)))
    # 1 = tests ran and some failed (not a crash, a collection error or an empty run)
    assert r.returncode == 1, f"{name}: pins did not fail (rc {r.returncode})\n" + r.stdout[-2000:]
    assert " failed" in r.stdout


PY_MUTANTS = {
    # D4 treated as abelian: the reflection does not reverse the rotation
    "d4_product_abelian": ("dihedral.py", "return index(a + (c if b == 0 else -c), b + d)",
                           "return index(a + c, b + d)"),
    "d4_rotation_not_inverted": ("dihedral.py", "return index(-a, 0) if b == 0 else g",
                                 "return index(a, 0) if b == 0 else g"),
    "d4_layer_reads_h_ginv": ("dihedral.py", "idx = np.array([[mul(inv(g), h) for g",
                              "idx = np.array([[mul(h, inv(g)) for g"),
    "d4_dw_folded_on_ginv_h_swapped": ("dihedral.py", "dW[:, :, mul(inv(g), h)] += dE[:, h, :, g]",
                                       "dW[:, :, mul(inv(h), g)] += dE[:, h, :, g]"),
    "d4_character_table": ("dihedral.py", "(1, (-1) ** b, (-1) ** a, (-1) ** (a + b))",
                           "(1, (-1) ** b, (-1) ** a, (-1) ** a)"),
    "d4_irrep_factor_order": ("dihedral.py", "np.linalg.matrix_power(_R, a) @ np.linalg.matrix_power(_S, b)",
                              "np.linalg.matrix_power(_S, b) @ np.linalg.matrix_power(_R, a)"),
    "gelu_wrong_scale": ("__init__.py", "0.5 * v * (1.0 + erf(v / np.sqrt(2.0)))", "0.5 * v * (1.0 + erf(v / 2.0))"),
    "mlp_block_without_activation": ("__init__.py", "hidden = gelu(forward(x, W1, b1, threads))",
                                     "hidden = forward(x, W1, b1, threads)"),
    # the p4 group convolution: filter turned with R^h instead of R^-h
    "conv_filter_turned_forward": ("conv.py", "fy, fx = rotate_offset(dy, dx, -h)",
                                   "fy, fx = rotate_offset(dy, dx, h)"),
    "conv_group_index_reversed": ("conv.py", "w = psi[:, :, (h - g) % G, fy + r, fx + r]",
                                  "w = psi[:, :, (g - h) % G, fy + r, fx + r]"),
    # a convolution instead of a cross-correlation over the pixels
    "conv_offset_sign": ("conv.py", "xs = shifted(x, dy, dx)", "xs = shifted(x, -dy, -dx)"),
    "conv_rotation_inverted": ("conv.py", "dy, dx = -dx, dy", "dy, dx = dx, -dy"),
    "conv_bias_dropped": ("conv.py", "    if bias is not None:\n        y +=", "    if False:\n        y +="),
    "conv_zero_padding_wraps": ("conv.py", "        s[:, y0:y1, x0:x1] = x[:, y0 + dy:y1 + dy, x0 + dx:x1 + dx]",
                                "        s[:, y0:y1, x0:x1] = x[:, y0 + dy:y1 + dy, x0 + dx:x1 + dx]\n"
                                "        s = np.roll(x, (-dy, -dx), axis=(1, 2))"),
}


def _run_py_copy(tmp_path, edit=None):
    """pytest of the oracle pins in a child process whose ``oracle`` package is a copy (optionally
    with one edit); the C part is the normal build."""
    import oracle

    lib = oracle.build(force=False)
    root = tmp_path / "root"
    shutil.copytree(os.path.join(ROOT, "oracle"), root / "oracle", ignore=shutil.ignore_patterns("__pycache__", "_build"))
    (root / "tests").mkdir()
    for f in ("conftest.py", "test_oracle.py", "test_oracle_dihedral.py", "test_oracle_conv.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), root / "tests" / f)
    if edit:
        fname, old, new = edit
        path = root / "oracle" / fname
        text = path.read_text()
        assert text.count(old) == 1, f"anchor not unique in oracle/{fname}: {old}"
        path.write_text(text.replace(old, new))
    env = dict(os.environ, EQLIN_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    cmd = [sys.executable, "-m", "pytest", "tests", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
    return subprocess.run(cmd, cwd=str(root), env=env, capture_output=True, text=True, timeout=300)


def test_unmodified_python_copy_passes(tmp_path):
    r = _run_py_copy(tmp_path)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert " passed" in r.stdout


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_planted_python_mistake_is_caught(tmp_path, name):
    r = _run_py_copy(tmp_path, PY_MUTANTS[name])
    assert r.returncode == 1, f"{name}: pins did not fail (rc {r.returncode})\n" + r.stdout[-2000:]
    assert " failed" in r.stdout
