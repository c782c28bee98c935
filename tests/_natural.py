"""Other valid implementations of the FFN chain, used only to measure how far
correct implementations drift apart in a free-running FP8 chain.

Each is the oracle's chain with one change: every GEMM sums the (exact) FP8
products in fp32, in one of several orders, instead of exactly.  The method
asks for an fp32-accumulated GEMM and leaves the order open, so each is as
correct as the oracle.  Their distances from the oracle after L layers (1 -
cosine of Z) spread widely, because an FP8 chain is chaotic: once one code
flips near a rounding boundary, the difference grows layer by layer.  The
GPU's free-running chain is judged against that spread.

Orders:
  blas      the host BLAS's float32 matmul (its own blocking)
  blas_rev  the same over the reversed K order
  split4    four K quarters summed by BLAS, then added in fp32 in order
  seq16     exact sums of 16 consecutive products added one after another
            into an fp32 accumulator (the matrix cores' per-instruction sums
            accumulated along K, as the GPU's GEMMs do)
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


def _mm_blas(X, W):
    return X @ W.T


def _mm_rev(X, W):
    return np.ascontiguousarray(X[:, ::-1]) @ np.ascontiguousarray(W[:, ::-1]).T


def _mm_split4(X, W):
    q = X.shape[1] // 4
    acc = None
    for s in range(4):
        p = X[:, s * q:(s + 1) * q] @ W[:, s * q:(s + 1) * q].T
        acc = p if acc is None else (acc + p).astype(np.float32)
    return acc


def _mm_seq16(X, W):
    Xd = X.astype(np.float64)
    Wd = W.astype(np.float64)
    acc = np.zeros((X.shape[0], W.shape[0]), np.float32)
    for c in range(0, X.shape[1], 16):
        ch = Xd[:, c:c + 16] @ Wd[:, c:c + 16].T  # exact: 16 E4M3 products
        acc = (acc.astype(np.float64) + ch).astype(np.float32)
    return acc


ORDERS = {"blas": _mm_blas, "blas_rev": _mm_rev, "split4": _mm_split4, "seq16": _mm_seq16}


def block_fp32_sums(r, y, lw: oracle.LayerWeights, act: int, eps: float, s_x: float, s_h: float,
                    order: str = "blas"):
    mm = ORDERS[order]
    L8 = lut()
    inv_x = np.float32(np.float32(1.0) / np.float32(s_x))
    inv_h = np.float32(np.float32(1.0) / np.float32(s_h))
    r1, _, xq = oracle.add_rmsnorm_quant(r, y, lw.w_norm, eps, inv_x, mod=lw.mod)
    X = L8[xq]
    Au = mm(X, L8[lw.qu])
    Ag = None if lw.qg is None else mm(X, L8[lw.qg])
    a_g = np.float32(np.float32(s_x) * np.float32(lw.s_g))
    a_u = np.float32(np.float32(s_x) * np.float32(lw.s_u))
    _, hq = oracle.gateup_epilogue(Ag, Au, act, a_g, a_u, inv_h)
    Ad = mm(L8[hq], L8[lw.qd])
    y1 = oracle.down_epilogue(Ad, np.float32(np.float32(s_h) * np.float32(lw.s_d)))
    return r1, y1


class NaturalChains:
    """The chain in every order, stepped layer by layer beside the oracle."""

    def __init__(self, r0, y0, orders=tuple(ORDERS)):
        self.state = {o: (r0, y0) for o in orders}

    def step(self, lw, act, eps, s_x, s_h):
        for o, (r, y) in self.state.items():
            self.state[o] = block_fp32_sums(r, y, lw, act, eps, s_x, s_h, o)

    def distances(self, z_ref) -> dict:
        return {o: cos_distance(oracle.final_hidden(r, y), z_ref) for o, (r, y) in self.state.items()}


def cos_distance(a_bits, b_bits) -> float:
    a = oracle.bf16_to_f32(a_bits).astype(np.float64).ravel()
    b = oracle.bf16_to_f32(b_bits).astype(np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 or nb == 0:
        return 0.0 if na == nb else 1.0
    return float(1.0 - a @ b / (na * nb))
