"""Build libfrt.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Flags: -ffp-contract=off keeps every rounding point as written in the
kernels; packed fp32 instructions are disabled for all device code.  Each
source compiles to its own object (in parallel) under _build/, then one link
makes the shared library.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfrt.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["frt_ffn.hip", "frt_qkv.hip", "k_norm.hip", "k_quant.hip", "k_gemm.hip", "k_mm.hip", "k_calib.hip",
           "k_qkv.hip", "k_mx.hip", "k_mxmm.hip"]
HEADERS = ["frt_device.h", "frt_host.h", "frt_qkv_dev.h", "frt_mx.h", os.path.join("..", "..", "include", "frt_ffn.h"),
           os.path.join("..", "..", "include", "frt_qkv.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    return "hipcc"


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(CSRC, h) for h in HEADERS]
    return any(os.path.getmtime(d) > t for d in deps if os.path.exists(d))


def _compile(src: str) -> tuple:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + HIPCC_FLAGS + ["-c", "-o", obj, os.path.join(CSRC, src)]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return obj, res.returncode, res.stdout


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every source into libfrt.so (always when force, else only if stale)."""
    if not force and not stale():
        return LIB
    os.makedirs(BUILD_DIR, exist_ok=True)
    try:
        workers = max(1, min(len(SOURCES), len(os.sched_getaffinity(0)), 8))
    except AttributeError:  # pragma: no cover
        workers = 4
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(_compile, SOURCES))
    bad = [(o, out) for o, rc, out in results if rc != 0]
    if bad:
        raise RuntimeError("hipcc failed:\n" + "\n".join(out for _, out in bad))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _, _ in results]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + res.stdout)
    if verbose:
        print("\n".join(out for _, _, out in results) + res.stdout)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True))
