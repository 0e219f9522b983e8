"""The oracle's pins must catch plausible mistakes: each case below plants one slip in a copy of
oracle/eqlin_oracle.c (a wrong index, a sign, a dropped term or bias), builds it, and runs
tests/test_oracle.py against that build in a child process, which must then fail. An unmodified
copy built the same way must pass, so a failure is the pins' doing and not the harness's. Every
slip keeps all memory accesses in bounds."""
import os
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
