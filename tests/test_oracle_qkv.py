"""Pins of the oracle's attention-input path (FlashRT architecture doc,
"Kernel library": the "qkv split + RoPE" fusion; itsolotime article section
5.2: the FusedQKV weight): the rotary table against closed forms, the
rotation's pairing, sign and identity cases, the head split, the shared
per-tensor weight scale, and the block's wiring through unit weights."""
import math

import numpy as np
import pytest

import oracle

COS1 = 0.5403023058681398  # cos(1 rad)
SIN1 = 0.8414709848078965  # sin(1 rad)


def _bf16(x):
    return oracle.bf16_round(np.asarray(x, np.float32))


def test_table_position_zero_is_identity():
    t = oracle.rope_table(3, 64, 10000.0)
    assert t.shape == (3, 32, 2)
    assert np.all(t[0, :, 0] == 1.0) and np.all(t[0, :, 1] == 0.0)


@pytest.mark.parametrize("hd,base,p,i", [
    (64, 10000.0, 1, 0),        # theta_0 = 1
    (256, 10000.0, 100, 64),    # theta = 10000^(-1/2) = 0.01
    (128, 10000.0, 100, 32),
    (128, 1e6, 1000, 32),       # theta = 1e6^(-1/2) = 0.001
])
def test_table_hits_one_radian(hd, base, p, i):
    t = oracle.rope_table(p + 1, hd, base)
    assert t[p, i, 0] == np.float32(COS1) and t[p, i, 1] == np.float32(SIN1)


def test_table_quarter_index_differs_from_wrong_exponent():
    # with exponent -i/hd instead of -2i/hd, index hd/4 would be base^(-1/4)
    t = oracle.rope_table(11, 128, 10000.0)
    assert abs(float(t[10, 32, 0]) - math.cos(0.1)) < 1e-7  # 10 * 0.01 rad
    assert abs(float(t[10, 32, 0]) - math.cos(1.0)) > 0.1


def test_table_is_on_the_unit_circle():
    t = oracle.rope_table(257, 128, 1e6).astype(np.float64)
    r = t[..., 0] ** 2 + t[..., 1] ** 2
    assert np.max(np.abs(r - 1)) < 2.0 ** -22


def _A(seed, M, nq, nkv, hd, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, (nq + 2 * nkv) * hd)) * scale).astype(np.float32)


def test_position_zero_gives_dequantised_split():
    M, nq, nkv, hd = 3, 4, 2, 64
    A = _A(1, M, nq, nkv, hd)
    alpha = np.float32(0.37)
    t = oracle.rope_table(8, hd, 10000.0)
    q, k, v = oracle.qkv_epilogue(A, alpha, nq, nkv, hd, np.zeros(M, np.int32), t)
    ref = _bf16(A * alpha)  # f32 product, then bf16
    assert np.array_equal(q.reshape(M, -1), ref[:, :nq * hd])
    assert np.array_equal(k.reshape(M, -1), ref[:, nq * hd:(nq + nkv) * hd])
    assert np.array_equal(v.reshape(M, -1), ref[:, (nq + nkv) * hd:])


def test_half_split_pairing_with_one_hot_input():
    # only dimension 0 of head 0 is set: its partner is dimension hd/2
    M, nq, nkv, hd = 1, 2, 1, 64
    A = np.zeros((M, (nq + 2 * nkv) * hd), np.float32)
    A[0, 0] = 1.5
    t = oracle.rope_table(2, hd, 10000.0)  # position 1, index 0: 1 radian
    q, k, v = oracle.qkv_epilogue(A, 1.0, nq, nkv, hd, np.array([1], np.int32), t)
    exp = np.zeros(hd, np.uint16)
    exp[0] = _bf16([np.float32(1.5) * np.float32(COS1)])[0]
    exp[hd // 2] = _bf16([np.float32(1.5) * np.float32(SIN1)])[0]
    assert np.array_equal(q[0, 0], exp)
    assert not np.any(q[0, 1]) and not np.any(k) and not np.any(v)
    assert q[0, 0, 1] == 0  # an adjacent-pair rotation would put the sine term here


def test_quarter_turn_signs_with_a_hand_made_table():
    # cos = 0, sin = 1 everywhere: out[d] = -x[d+hd/2], out[d+hd/2] = x[d]
    M, nq, nkv, hd = 2, 1, 1, 32
    A = _bf16(_A(3, M, nq, nkv, hd)).view(np.uint16)
    Af = oracle.bf16_to_f32(A)  # bf16-exact values: the products round exactly
    t = np.zeros((4, hd // 2, 2), np.float32)
    t[..., 1] = 1.0
    q, k, _ = oracle.qkv_epilogue(Af, 1.0, nq, nkv, hd, np.array([3, 2], np.int32), t)
    for out, base in ((q[:, 0], 0), (k[:, 0], hd)):
        x = Af[:, base:base + hd]
        assert np.array_equal(out[:, :hd // 2], _bf16(-x[:, hd // 2:]))
        assert np.array_equal(out[:, hd // 2:], _bf16(x[:, :hd // 2]))


def test_rotation_keeps_pair_length_and_relative_position():
    M, nq, nkv, hd = 1, 1, 1, 128
    rng = np.random.default_rng(9)
    A = rng.standard_normal((M, 3 * hd)).astype(np.float32)
    t = oracle.rope_table(600, hd, 10000.0)

    def rot(p):
        q, k, _ = oracle.qkv_epilogue(A, 1.0, nq, nkv, hd, np.array([p], np.int32), t)
        return oracle.bf16_to_f32(q[0, 0]).astype(np.float64), oracle.bf16_to_f32(k[0, 0]).astype(np.float64)

    q0, k0 = rot(0)
    q5, _ = rot(5)
    h = hd // 2
    assert np.allclose(q5[:h] ** 2 + q5[h:] ** 2, q0[:h] ** 2 + q0[h:] ** 2, rtol=2e-2, atol=1e-3)
    # <R(m) q, R(n) k> depends on m - n only
    qa, _ = rot(17)
    _, kb = rot(10)
    qc, _ = rot(517)
    _, kd = rot(510)
    assert abs(qa @ kb - qc @ kd) < 2e-2 * (np.linalg.norm(q0) * np.linalg.norm(k0))


def test_position_outside_table_is_rejected():
    A = _A(4, 1, 1, 1, 32)
    with pytest.raises(ValueError):
        oracle.qkv_epilogue(A, 1.0, 1, 1, 32, np.array([4], np.int32), oracle.rope_table(4, 32, 1e4))


def test_fused_weight_has_one_scale_for_all_three():
    rng = np.random.default_rng(5)
    H, hd = 64, 32
    wq = _bf16(rng.standard_normal((2 * hd, H)) * 0.02)
    wk = _bf16(rng.standard_normal((hd, H)) * 0.02)
    wv = _bf16(rng.standard_normal((hd, H)) * 0.02)
    wk[3, 7] = _bf16([0.5])[0]  # the largest magnitude sits in K
    qw = oracle.QkvWeights.quantize(wq, wk, wv, np.full(H, oracle.ONES_BF16, np.uint16), hd)
    assert qw.s_w == np.float32(np.float32(0.5) / np.float32(448.0))
    assert qw.codes.shape == (4 * hd, H)
    assert qw.codes[2 * hd + 3, 7] == 0x7E  # +448
    assert (qw.nq, qw.nkv, qw.hd) == (2, 1, hd)


def test_block_wiring_with_unit_weights():
    # code 0x38 = 1.0; row n of the fused weight picks input column n % H, so
    # A[m][n] = dec(xq[m][n % H]) and at position 0 every output is
    # bf16(f32(dec(xq) * alpha))
    rng = np.random.default_rng(6)
    M, H, nq, nkv, hd = 5, 128, 2, 1, 32
    N = (nq + 2 * nkv) * hd
    r = _bf16(rng.standard_normal((M, H)))
    y = _bf16(rng.standard_normal((M, H)))
    codes = np.zeros((N, H), np.uint8)
    codes[np.arange(N), np.arange(N) % H] = 0x38
    qw = oracle.QkvWeights(codes, 0.25, np.full(H, oracle.ONES_BF16, np.uint16), nq, nkv, hd)
    s_x = 0.01
    t = oracle.rope_table(2, hd, 1e4)
    r_out, xq, q, k, v = oracle.qkv_block(r, y, qw, 1e-6, s_x, np.zeros(M, np.int32), t)
    inv_x = np.float32(np.float32(1.0) / np.float32(s_x))
    r_ref, _, xq_ref = oracle.add_rmsnorm_quant(r, y, qw.w_norm, 1e-6, float(inv_x))
    assert np.array_equal(r_out, r_ref) and np.array_equal(xq, xq_ref)
    alpha = np.float32(np.float32(s_x) * np.float32(0.25))
    vals = _bf16(oracle.e4m3_decode(xq).astype(np.float32)[:, np.arange(N) % H] * alpha)
    assert np.array_equal(q.reshape(M, -1), vals[:, :nq * hd])
    assert np.array_equal(k.reshape(M, -1), vals[:, nq * hd:(nq + nkv) * hd])
    assert np.array_equal(v.reshape(M, -1), vals[:, (nq + nkv) * hd:])


def test_calibration_is_brute_force_max():
    rng = np.random.default_rng(7)
    M, H, hd = 4, 64, 32
    wn = _bf16(1 + 0.1 * rng.standard_normal(H))
    qw = oracle.QkvWeights.quantize(_bf16(rng.standard_normal((hd, H))), _bf16(rng.standard_normal((hd, H))),
                                    _bf16(rng.standard_normal((hd, H))), wn, hd)
    batches = [(_bf16(rng.standard_normal((M, H))), None) for _ in range(3)]
    s = oracle.qkv_calibrate(batches, qw, 1e-6)
    amax = 0.0
    for rr, _ in batches:
        _, x, _ = oracle.add_rmsnorm_quant(rr, None, wn, 1e-6, 1.0)
        amax = max(amax, float(np.abs(x).max()))
    assert s == np.float32(np.float32(amax) / np.float32(448.0))
