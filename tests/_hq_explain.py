"""Is an HQ code mismatch explained by fp32 accumulation error?

The re-quantised activation HQ is formed from fp32 GEMM accumulators.  The
method fixes "fp32 accumulate" but not the order of the sum, so a correct
kernel's accumulator differs from the oracle's exact sum rounded once, and an
element whose exact value sits close to an E4M3 rounding boundary may round
to the neighbouring code.  This module measures, for each mismatched element,
how large an accumulation error would be needed to produce the GPU's code.

Unit of error.  Summing K products p_k one after another in fp32 makes K
roundings, the k-th of size at most u|S_k| (u = 2^-24, S_k the partial sum);
with the partial sums of a random walk the standard deviation of the total
error is about 0.2 u sqrt(K) sqrt(sum_k p_k^2) (each rounding uniform on
[-u/2, u/2] |S_k|, E S_k^2 = k mean(p^2)).  The unit used here is
E = u sqrt(K) Q with Q = sqrt(sum_k p_k^2), i.e. about five of those standard
deviations; any shorter summation tree (split-K, per-instruction sums) has a
smaller error.  The GPU's activation function adds a relative error of its
own (hardware exp2 / reciprocal approximations, below 2e-6); ACT_SLACK covers
it.

For each mismatch the search finds the smallest t such that some accumulator
pair (A_g + s_g t E_g, A_u + s_u t E_u), s = +-1, run through the oracle's own
epilogue (and a relative ACT_SLACK on h), yields the GPU's code.  A correct
fp32-accumulating kernel gives t well below 1; a kernel whose products lose
bits inside the matrix instruction needs t of several units.
"""
from __future__ import annotations

import numpy as np

import oracle

U32 = 2.0 ** -24
ACT_SLACK = 2e-6
T_GRID = np.concatenate([[0.0], np.geomspace(1e-3, 64.0, 120)])
T_MAX_EXPLAINED = 2.0

_LUT = None


def _lut() -> np.ndarray:
    global _LUT
    if _LUT is None:
        v = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
        v[np.isnan(v)] = 0.0
        _LUT = v
    return _LUT


def _codes_with_slack(h: np.ndarray, inv_h: float) -> list:
    """E4M3 codes of f32(h * inv_h) and of h moved by +-ACT_SLACK relative."""
    out = []
    for f in (1.0, 1.0 + ACT_SLACK, 1.0 - ACT_SLACK):
        hv = (h.astype(np.float64) * f).astype(np.float32)
        out.append(oracle.e4m3_encode((hv * np.float32(inv_h)).astype(np.float32)))
    return out


def min_t(xq_row: np.ndarray, wg_row, wu_row: np.ndarray, act: int, alpha_g: float, alpha_u: float,
          inv_h: float, gpu_code: int) -> float:
    """Smallest error (in units E) that turns the oracle's code into gpu_code
    (inf if none up to the grid's end)."""
    lut = _lut()
    x = lut[xq_row]
    K = x.size
    pu = x * lut[wu_row]
    Au = float(np.sum(pu))  # exact: E4M3 products and their sums fit fp64 (K <= 2^15)
    Eu = U32 * np.sqrt(K) * float(np.sqrt(np.sum(pu * pu)))
    if wg_row is not None:
        pg = x * lut[wg_row]
        Ag = float(np.sum(pg))
        Eg = U32 * np.sqrt(K) * float(np.sqrt(np.sum(pg * pg)))
    nt = T_GRID.size
    cand_u, cand_g = [], []
    for su in (1.0, -1.0):
        for sg in ((1.0, -1.0) if wg_row is not None else (0.0,)):
            cand_u.append(Au + su * T_GRID * Eu)
            if wg_row is not None:
                cand_g.append(Ag + sg * T_GRID * Eg)
    a_u = np.concatenate(cand_u).astype(np.float32)
    a_g = None if wg_row is None else np.concatenate(cand_g).astype(np.float32)
    h, _ = oracle.gateup_epilogue(a_g, a_u, act, alpha_g, alpha_u, inv_h)
    hit = np.zeros(h.size, bool)
    for codes in _codes_with_slack(h, inv_h):
        hit |= codes == gpu_code
    hit = hit.reshape(-1, nt)
    best = np.inf
    for row in hit:
        idx = np.flatnonzero(row)
        if idx.size:
            best = min(best, float(T_GRID[idx[0]]))
    return best


def explain(xq: np.ndarray, hq_gpu: np.ndarray, hq_ref: np.ndarray, lw, act: int, s_x: float,
            s_h: float) -> tuple:
    """-> (number of mismatches, largest t over them) for one layer's
    teacher-forced HQ; xq are the oracle's (= the GPU's) activation codes."""
    bad = np.argwhere(hq_gpu != hq_ref)
    if bad.size == 0:
        return 0, 0.0
    alpha_g = float(np.float32(np.float32(s_x) * np.float32(lw.s_g)))
    alpha_u = float(np.float32(np.float32(s_x) * np.float32(lw.s_u)))
    inv_h = float(np.float32(np.float32(1.0) / np.float32(s_h)))
    tmax = 0.0
    for r, i in bad:
        t = min_t(xq[r], None if lw.qg is None else lw.qg[i], lw.qu[i], act, alpha_g, alpha_u, inv_h,
                  int(hq_gpu[r, i]))
        tmax = max(tmax, t)
    return int(bad.shape[0]), tmax
