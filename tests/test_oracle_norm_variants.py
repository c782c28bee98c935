"""Pins of the oracle's norm variants (itsolotime article, section 5.2):
Pi0-style norm fusion (the RMSNorm weight folded into the gate/up matrices
per input column before quantisation) and Pi0.5-style AdaRMSNorm modulation
(x = t * (1 + scale) + shift instead of t * w).  Each variant is tied to the
already-pinned plain path by an exact reduction, plus an orientation check
that a transposed fold fails."""
import numpy as np

import oracle

EPS = np.float32(1e-6)


def _bf16(x):
    return oracle.bf16_round(np.asarray(x, np.float32))


def _rows(seed, M, H):
    rng = np.random.default_rng(seed)
    return _bf16(rng.standard_normal((M, H)).astype(np.float32)), _bf16(rng.standard_normal((M, H)).astype(np.float32))


def _weight_and_scale_minus_one(seed, H):
    """w in [0.5, 2) as bf16, and scale = w - 1, exact in bf16, with
    f32(1 + scale) == w exactly (asserted)."""
    rng = np.random.default_rng(seed)
    w = _bf16(rng.uniform(0.5, 2.0, H).astype(np.float32))
    wf = oracle.bf16_to_f32(w).astype(np.float64)
    sc = _bf16((wf - 1.0).astype(np.float32))
    assert np.array_equal(oracle.bf16_to_f32(sc).astype(np.float64), wf - 1.0)
    assert np.array_equal((np.float32(1.0) + oracle.bf16_to_f32(sc)).astype(np.float32), oracle.bf16_to_f32(w))
    return w, sc


def test_ada_with_scale_w_minus_one_equals_weighted_norm():
    M, H = 7, 384
    r, y = _rows(11, M, H)
    w, sc = _weight_and_scale_minus_one(12, H)
    zero = np.zeros(H, np.uint16)
    inv_x = np.float32(1.0 / 0.013)
    r1, x1, q1 = oracle.add_rmsnorm_quant(r, y, w, EPS, inv_x)
    r2, x2, q2 = oracle.add_rmsnorm_quant(r, y, np.zeros(H, np.uint16), EPS, inv_x, mod=(sc, zero))
    assert np.array_equal(r1, r2)
    assert np.array_equal(x1, x2)
    assert np.array_equal(q1, q2)


def test_ada_identity_modulation_equals_unit_weight():
    M, H = 5, 256
    r, y = _rows(21, M, H)
    ones = np.full(H, oracle.ONES_BF16, np.uint16)
    zero = np.zeros(H, np.uint16)
    _, x1, q1 = oracle.add_rmsnorm_quant(r, y, ones, EPS, 3.0)
    _, x2, q2 = oracle.add_rmsnorm_quant(r, y, ones, EPS, 3.0, mod=(zero, zero))
    assert np.array_equal(x1, x2) and np.array_equal(q1, q2)


def test_ada_scale_minus_one_leaves_only_the_shift():
    # 1 + (-1) = 0 exactly, so x = t * 0 + shift = shift for every element
    M, H = 4, 128
    r, y = _rows(31, M, H)
    rng = np.random.default_rng(32)
    shift = _bf16(rng.standard_normal(H).astype(np.float32) * 3)
    minus_one = np.full(H, 0xBF80, np.uint16)
    _, x, _ = oracle.add_rmsnorm_quant(r, y, np.zeros(H, np.uint16), EPS, 1.0, mod=(minus_one, shift))
    assert np.array_equal(x, np.broadcast_to(oracle.bf16_to_f32(shift), (M, H)))


def test_ada_shift_moves_the_quantiser_input():
    # the shift enters after the scale: shift = c with scale = -1 and a
    # quantiser factor inv_x gives e4m3(c * inv_x) in every position
    M, H = 3, 64
    r, y = _rows(41, M, H)
    c = _bf16(np.full(H, 0.75, np.float32))
    _, _, q = oracle.add_rmsnorm_quant(r, y, np.zeros(H, np.uint16), EPS, 8.0,
                                       mod=(np.full(H, 0xBF80, np.uint16), c))
    assert np.all(q == oracle.e4m3_encode(np.float32(6.0)))


def test_fold_with_unit_column_factor_is_plain_quantisation():
    rng = np.random.default_rng(51)
    W = _bf16(rng.standard_normal((48, 96)).astype(np.float32) * 0.02)
    ones = np.full(96, oracle.ONES_BF16, np.uint16)
    c1, s1 = oracle.quant_tensor(W)
    c2, s2 = oracle.quant_tensor_fold(W, ones)
    assert s1 == s2 and np.array_equal(c1, c2)


def test_fold_scales_input_columns_not_rows():
    # W = all ones [rows][cols] with distinct column factors: every row of the
    # folded tensor is the factor vector, so every row's codes equal the
    # quantisation of that vector alone (a row-wise fold would give constant rows)
    rows, cols = 5, 72
    rng = np.random.default_rng(61)
    colw = _bf16(rng.uniform(0.5, 1.5, cols).astype(np.float32))
    W = np.full((rows, cols), oracle.ONES_BF16, np.uint16)
    codes, s = oracle.quant_tensor_fold(W, colw)
    ref, s_ref = oracle.quant_tensor(colw[None, :])
    assert s == s_ref
    assert np.array_equal(codes, np.broadcast_to(ref, (rows, cols)))
    assert len(np.unique(codes[0])) > 1


def test_fold_by_power_of_two_keeps_codes_and_scales_the_scale():
    rng = np.random.default_rng(71)
    W = _bf16(rng.standard_normal((32, 64)).astype(np.float32) * 0.02)
    four = _bf16(np.full(64, 4.0, np.float32))
    c1, s1 = oracle.quant_tensor(W)
    c2, s2 = oracle.quant_tensor_fold(W, four)
    assert np.array_equal(c1, c2)
    assert s2 == np.float32(4.0) * np.float32(s1)


def test_norm_fuse_layer_uses_unit_norm_weight_and_folded_codes():
    rng = np.random.default_rng(81)
    H, I = 64, 96
    wg = _bf16(rng.standard_normal((I, H)).astype(np.float32) * 0.02)
    wu = _bf16(rng.standard_normal((I, H)).astype(np.float32) * 0.02)
    wd = _bf16(rng.standard_normal((H, I)).astype(np.float32) * 0.02)
    wn = _bf16(1 + 0.1 * rng.standard_normal(H).astype(np.float32))
    lw = oracle.LayerWeights.quantize(wg, wu, wd, wn, norm_fuse=True)
    assert np.all(lw.w_norm == oracle.ONES_BF16)
    assert np.array_equal(lw.qg, oracle.quant_tensor_fold(wg, wn)[0])
    assert np.array_equal(lw.qu, oracle.quant_tensor_fold(wu, wn)[0])
    assert np.array_equal(lw.qd, oracle.quant_tensor(wd)[0])  # the down matrix is not folded


def test_ada_calibration_is_brute_force_max():
    rng = np.random.default_rng(91)
    M, H, I = 6, 64, 128
    wg = _bf16(rng.standard_normal((I, H)).astype(np.float32) * 0.02)
    wu = _bf16(rng.standard_normal((I, H)).astype(np.float32) * 0.02)
    wd = _bf16(rng.standard_normal((H, I)).astype(np.float32) * 0.02)
    wn = _bf16(np.ones(H, np.float32))
    sc = _bf16(0.2 * rng.standard_normal(H).astype(np.float32))
    sh = _bf16(0.2 * rng.standard_normal(H).astype(np.float32))
    lw = oracle.LayerWeights.quantize(wg, wu, wd, wn, mod=(sc, sh))
    r, y = _rows(92, M, H)
    _, _, ax, _ = oracle.block_measure(r, y, lw, 0, float(EPS))
    _, x, _ = oracle.add_rmsnorm_quant(r, y, wn, EPS, 1.0, mod=(sc, sh))
    assert ax == float(np.max(np.abs(x)))
