"""The packed weight orders (MFMA fragment order, the decode GEMVs' column
quads and octets, the fused QKV pairs and octets, the MXFP4 GEMV and
column-quad orders) checked on the host: a
small program built with hipcc from the same headers the kernels and the
export paths use (tests/layouts/layout_check.hip) verifies that every order
is a bijection and keeps together what its kernel needs together.  No GPU is
used."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "layouts", "layout_check.hip")
CSRC = os.path.join(ROOT, "realtime_transformer_amd", "csrc")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_packed_orders_are_bijections():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "layout_check")
        b = subprocess.run([hipcc, "-O1", "-std=c++17", "-I", CSRC, "-o", exe, SRC], capture_output=True, text=True)
        assert b.returncode == 0, b.stdout + b.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "layout checks ok" in r.stdout
