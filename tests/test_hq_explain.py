"""Pins of the HQ mismatch analysis (tests/_hq_explain.py) on the CPU.

A plainly valid fp32 accumulation (one product after another, the longest
summation chain and the largest rounding error any order has) must have every
one of its HQ mismatches explained; accumulators that lose bits the way a
truncating adder does (a relative error of ~1e-4 to 1e-3) must not be.
"""
import numpy as np
import pytest

import oracle
from realtime_transformer_amd import datagen
from realtime_transformer_amd.configs import FFNConfig, ACT_GEGLU_TANH, ACT_GELU_TANH

import _hq_explain


def _layer(idx, M, H, I, act):
    cfg = FFNConfig(idx, "hqx_%d" % idx, M, H, I, 1, act)
    wg, wu, wd, wn = datagen.layer_weights(cfg, 0)
    lw = oracle.LayerWeights.quantize(wg, wu, wd, wn)
    r0, _ = datagen.eval_inputs(cfg)
    _, x, _ = oracle.add_rmsnorm_quant(r0, None, lw.w_norm, cfg.eps, 1.0)
    s_x = oracle.scale_from_amax(float(np.max(np.abs(x))))
    inv_x = np.float32(np.float32(1.0) / np.float32(s_x))
    _, _, xq = oracle.add_rmsnorm_quant(r0, None, lw.w_norm, cfg.eps, float(inv_x))
    return cfg, lw, xq, s_x


def _sequential_f32(X, W):
    """fp32 sum in K order, one rounding per product added."""
    acc = np.zeros((X.shape[0], W.shape[0]), np.float32)
    for k in range(X.shape[1]):
        acc = (acc + np.outer(X[:, k], W[:, k]).astype(np.float32)).astype(np.float32)
    return acc


def test_sequential_fp32_mismatches_are_explained():
    act = ACT_GELU_TANH
    cfg, lw, xq, s_x = _layer(902, 128, 4096, 4096, act)
    lut = _hq_explain._lut()
    X = lut[xq]
    W = lut[lw.qu]
    Au = _sequential_f32(X.astype(np.float32), W.astype(np.float32))
    exact = X @ W.T  # exact in fp64 (E4M3 products, K <= 2^15)
    # the error unit: the worst sequential-fp32 error over half a million
    # sums stays within T_MAX_EXPLAINED units, the typical one is far below
    E = _hq_explain.U32 * np.sqrt(X.shape[1]) * np.sqrt((X * X) @ (W * W).T)
    z = np.abs(Au.astype(np.float64) - exact) / E
    assert np.max(z) <= _hq_explain.T_MAX_EXPLAINED, np.max(z)
    assert 1e-3 < np.median(z) < 0.5, np.median(z)
    a_u = np.float32(np.float32(s_x) * np.float32(lw.s_u))
    h_ref, _ = oracle.gateup(xq, None, lw.qu, act, 1.0, a_u, 1.0)
    s_h = oracle.scale_from_amax(float(np.max(np.abs(h_ref))))
    inv_h = np.float32(np.float32(1.0) / np.float32(s_h))
    _, hq_ref = oracle.gateup(xq, None, lw.qu, act, 1.0, a_u, inv_h)
    _, hq_seq = oracle.gateup_epilogue(None, Au, act, 1.0, a_u, inv_h)
    n, tmax = _hq_explain.explain(xq, hq_seq, hq_ref, lw, act, s_x, s_h)
    # the sequential order does flip a code here, and it is explained
    assert n >= 1
    assert tmax <= _hq_explain.T_MAX_EXPLAINED, tmax


def test_lossy_accumulators_are_not_explained():
    act = ACT_GEGLU_TANH
    cfg, lw, xq, s_x = _layer(910, 64, 1024, 2048, act)
    lut = _hq_explain._lut()
    X = lut[xq]
    Ag = X @ lut[lw.qg].T
    Au = X @ lut[lw.qu].T
    a_g = np.float32(np.float32(s_x) * np.float32(lw.s_g))
    a_u = np.float32(np.float32(s_x) * np.float32(lw.s_u))
    h_ref, hq_ref = oracle.gateup_epilogue(Ag.astype(np.float32), Au.astype(np.float32), act, a_g, a_u, 1.0)
    s_h = oracle.scale_from_amax(float(np.max(np.abs(h_ref))))
    inv_h = np.float32(np.float32(1.0) / np.float32(s_h))
    _, hq_ref = oracle.gateup_epilogue(Ag.astype(np.float32), Au.astype(np.float32), act, a_g, a_u, inv_h)
    # a truncating adder: every accumulator moved toward zero by 3e-4 of itself
    lossy = (1.0 - 3e-4)
    _, hq_bad = oracle.gateup_epilogue((Ag * lossy).astype(np.float32), (Au * lossy).astype(np.float32), act,
                                       a_g, a_u, inv_h)
    n, tmax = _hq_explain.explain(xq, hq_bad, hq_ref, lw, act, s_x, s_h)
    assert n >= 20
    assert tmax > _hq_explain.T_MAX_EXPLAINED, tmax


def test_two_step_code_is_never_explained_by_small_errors():
    act = ACT_GEGLU_TANH
    cfg, lw, xq, s_x = _layer(911, 4, 512, 512, act)
    a_g = np.float32(np.float32(s_x) * np.float32(lw.s_g))
    a_u = np.float32(np.float32(s_x) * np.float32(lw.s_u))
    h_ref, _ = oracle.gateup(xq, lw.qg, lw.qu, act, a_g, a_u, 1.0)
    s_h = oracle.scale_from_amax(float(np.max(np.abs(h_ref))))
    inv_h = np.float32(np.float32(1.0) / np.float32(s_h))
    _, hq_ref = oracle.gateup(xq, lw.qg, lw.qu, act, a_g, a_u, inv_h)
    # pick an element with a large code and move its code two steps
    r, i = np.unravel_index(np.argmax(hq_ref & 0x7F), hq_ref.shape)
    bad = hq_ref.copy()
    bad[r, i] = (bad[r, i] & 0x80) | ((bad[r, i] & 0x7F) - 2)
    n, tmax = _hq_explain.explain(xq, bad, hq_ref, lw, act, s_x, s_h)
    assert n == 1 and tmax > _hq_explain.T_MAX_EXPLAINED
