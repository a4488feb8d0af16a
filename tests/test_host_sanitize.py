"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the library's host-side table builders (rns_ckks_polynomial_amd/csrc/
host_tables.cpp, checked against their definitions by tests/native/
host_tables_check.cpp) and the C oracle (every entry point, driven by
tests/native/oracle_sanitize_main.c).  Both are built with the host
compilers only; no GPU code is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(tmp_path, compiler, sources, extra, name):
    if not shutil.which(compiler):
        pytest.skip(f"{compiler} not available")
    exe = str(tmp_path / name)
    subprocess.run([compiler, *SAN, *extra, "-o", exe, *[os.path.join(ROOT, s) for s in sources], "-lm"],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


def test_host_tables_under_sanitizers(tmp_path):
    out = _run(tmp_path, "g++", ["tests/native/host_tables_check.cpp", "rns_ckks_polynomial_amd/csrc/host_tables.cpp"],
               ["-std=c++17"], "host_tables_check")
    assert out.count(": ok") == 4, out


def test_oracle_under_sanitizers(tmp_path):
    out = _run(tmp_path, "gcc", ["tests/native/oracle_sanitize_main.c", "oracle/oracle.c"], ["-std=gnu11", "-fopenmp"],
               "oracle_sanitize")
    assert "ok" in out, out
