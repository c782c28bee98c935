"""A second valid implementation of the FFN chain, used only to measure how
far two correct implementations drift apart in a free-running FP8 chain.

It is the oracle's chain with one change: every GEMM sums the (exact) FP8
products in fp32 in the order of the host BLAS (numpy float32 matmul) instead
of exactly.  The method asks for an fp32-accumulated GEMM and leaves the order
open, so this is as correct as the oracle; their distance after L layers is
the natural drift against which the GPU's free-running chain is judged.
"""
from __future__ import annotations

import numpy as np

import oracle

_LUT = None


def lut() -> np.ndarray:
    global _LUT
    if _LUT is None:
        v = oracle.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float32)
        v[np.isnan(v)] = 0.0
        _LUT = v
    return _LUT


def block_fp32_sums(r, y, lw: oracle.LayerWeights, act: int, eps: float, s_x: float, s_h: float):
    L8 = lut()
    inv_x = np.float32(np.float32(1.0) / np.float32(s_x))
    inv_h = np.float32(np.float32(1.0) / np.float32(s_h))
    r1, _, xq = oracle.add_rmsnorm_quant(r, y, lw.w_norm, eps, inv_x, mod=lw.mod)
    X = L8[xq]
    Au = X @ L8[lw.qu].T
    Ag = None if lw.qg is None else X @ L8[lw.qg].T
    a_g = np.float32(np.float32(s_x) * np.float32(lw.s_g))
    a_u = np.float32(np.float32(s_x) * np.float32(lw.s_u))
    _, hq = oracle.gateup_epilogue(Ag, Au, act, a_g, a_u, inv_h)
    Ad = L8[hq] @ L8[lw.qd].T
    y1 = oracle.down_epilogue(Ad, np.float32(np.float32(s_h) * np.float32(lw.s_d)))
    return r1, y1


def cos_distance(a_bits, b_bits) -> float:
    a = oracle.bf16_to_f32(a_bits).astype(np.float64).ravel()
    b = oracle.bf16_to_f32(b_bits).astype(np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 or nb == 0:
        return 0.0 if na == nb else 1.0
    return float(1.0 - a @ b / (na * nb))
