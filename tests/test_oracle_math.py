"""Pins of the oracle's GEMM, RMSNorm, activations and weight quantiser
against closed forms, invariants, brute force and library routines."""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand_codes(rng, shape, max_exp_field=15):
    c = rng.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E  # no NaN codes
    return c


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 17), (3, 16, 33), (16, 17, 3), (17, 2, 128),
                                   (33, 33, 16), (4, 5, 1000)])
def test_gemm_matches_fp64_matmul(M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    a = _rand_codes(rng, (M, K))
    b = _rand_codes(rng, (N, K))
    got = oracle.gemm_e4m3(a, b, nthreads=3)
    da = torch.from_numpy(oracle.e4m3_decode(a))
    db = torch.from_numpy(oracle.e4m3_decode(b))
    ref = (da @ db.T).numpy()  # exact in fp64 for these sizes (see test below)
    assert np.array_equal(got, ref.astype(np.float32))
    # non-square shapes catch a transposed operand
    assert got.shape == (M, N)


def test_gemm_exact_on_long_rows():
    # K = 17408 (the largest contraction in the workloads): the int64 sum is
    # exact, so it equals an fp64 sum of exactly-representable products in a
    # different order (pairwise, numpy) whenever that sum is also exact; use
    # integer-valued codes so every partial sum is an exact small integer.
    rng = np.random.default_rng(7)
    K = 17408
    ints = np.array([0x38, 0xB8, 0x40, 0xC0, 0x00], np.uint8)  # 1, -1, 2, -2, 0
    a = ints[rng.integers(0, 5, size=(2, K))]
    b = ints[rng.integers(0, 5, size=(3, K))]
    got = oracle.gemm_e4m3(a, b)
    ref = oracle.e4m3_decode(a) @ oracle.e4m3_decode(b).T
    assert np.array_equal(got, ref.astype(np.float32))
    # and with full-range codes the result equals the correctly rounded exact
    # rational sum (python integers)
    a = _rand_codes(rng, (1, K))
    b = _rand_codes(rng, (1, K))
    ka = [int(round(v * 512)) for v in oracle.e4m3_decode(a[0])]
    kb = [int(round(v * 512)) for v in oracle.e4m3_decode(b[0])]
    exact = sum(x * y for x, y in zip(ka, kb))
    assert oracle.gemm_e4m3(a, b)[0, 0] == np.float32(math.ldexp(exact, -18))


def test_gemm_identity_selection():
    rng = np.random.default_rng(1)
    a = _rand_codes(rng, (5, 64))
    eye = np.zeros((64, 64), np.uint8)
    eye[np.arange(64), np.arange(64)] = 0x38  # 1.0
    out = oracle.gemm_e4m3(a, eye)
    assert np.array_equal(out, oracle.e4m3_decode(a).astype(np.float32))
    perm = rng.permutation(64)
    sel = np.zeros((64, 64), np.uint8)
    sel[np.arange(64), perm] = 0x38
    out = oracle.gemm_e4m3(a, sel)
    assert np.array_equal(out, oracle.e4m3_decode(a)[:, perm].astype(np.float32))


def _bf16(x):
    return oracle.bf16_round(np.asarray(x, np.float32))


def test_rmsnorm_constant_row_closed_form():
    H = 256
    eps = np.float32(1e-6)
    for c in (1.0, 0.5, 3.0, -2.0):
        r = _bf16(np.full((1, H), c))
        w = _bf16(np.ones(H))
        r_out, x, xq = oracle.add_rmsnorm_quant(r, None, w, eps, 1.0)
        inv_rms = np.float32(1.0 / math.sqrt(c * c + float(eps)))
        assert np.array_equal(r_out, r)
        assert np.all(x == np.float32(np.float32(c) * inv_rms))
    # c = 1: x = f32(1/sqrt(1.000001))
    r = _bf16(np.ones((1, 64)))
    _, x, _ = oracle.add_rmsnorm_quant(r, None, _bf16(np.ones(64)), np.float32(1e-6), 1.0)
    assert x[0, 0] == np.float32(1.0 / math.sqrt(1.0 + float(np.float32(1e-6))))


def test_rmsnorm_invariants():
    rng = np.random.default_rng(2)
    M, H = 7, 512
    r = _bf16(rng.standard_normal((M, H)))
    y = _bf16(rng.standard_normal((M, H)))
    w = _bf16(np.ones(H))
    tiny = np.float32(1e-30)
    r_out, x, _ = oracle.add_rmsnorm_quant(r, y, w, tiny, 1.0)
    # residual add: bf16(r + y)
    expect = _bf16(oracle.bf16_to_f32(r) + oracle.bf16_to_f32(y))
    assert np.array_equal(r_out, expect)
    ms = np.mean(x.astype(np.float64) ** 2, axis=1)
    assert np.all(np.abs(ms - 1.0) <= 4e-7)
    # power-of-two scaling of the input leaves the output unchanged (eps ~ 0)
    r2 = _bf16(oracle.bf16_to_f32(r_out) * 4.0)
    _, x2, _ = oracle.add_rmsnorm_quant(r2, None, w, tiny, 1.0)
    assert np.array_equal(x, x2)
    # the weight multiplies after the normalisation, elementwise
    w3 = _bf16(rng.standard_normal(H) * 0.1 + 1.0)
    _, x3, _ = oracle.add_rmsnorm_quant(r_out, None, w3, tiny, 1.0)
    assert np.array_equal(x3, (x * oracle.bf16_to_f32(w3)).astype(np.float32))
    # eps enters inside the square root: a large eps shrinks a unit row
    one = _bf16(np.ones((1, H)))
    _, xe, _ = oracle.add_rmsnorm_quant(one, None, w, np.float32(3.0), 1.0)
    assert xe[0, 0] == np.float32(1.0 / math.sqrt(1.0 + 3.0))


def test_rmsnorm_quantiser_uses_inv_x():
    rng = np.random.default_rng(4)
    r = _bf16(rng.standard_normal((3, 128)))
    w = _bf16(np.ones(128))
    inv_x = np.float32(1.0 / 0.01)
    _, x, xq = oracle.add_rmsnorm_quant(r, None, w, np.float32(1e-6), inv_x)
    assert np.array_equal(xq, oracle.e4m3_encode((x * inv_x).astype(np.float32)))


def test_activations_match_torch_fp64():
    z = np.concatenate([np.linspace(-12, 12, 20001), np.array([0.0, 1e-8, -1e-8, 30, -30, 80, -80])])
    zt = torch.from_numpy(z)
    g_ref = torch.nn.functional.gelu(zt, approximate="tanh").numpy()
    s_ref = torch.nn.functional.silu(zt).numpy()
    g = np.array([oracle.gelu_tanh(v) for v in z])
    s = np.array([oracle.silu(v) for v in z])
    # 1 + tanh(t) cancels for very negative z in any fp64 evaluation, so the
    # comparison is absolute at the scale of |z| * 2^-50 there
    tol = 1e-14 * np.abs(g_ref) + 1e-15 * np.maximum(1.0, np.abs(z))
    assert np.all(np.abs(g - g_ref) <= tol)
    assert np.allclose(s, s_ref, rtol=1e-14, atol=1e-300)
    # rounded once to fp32: within one fp32 ulp of the fp64 library value at
    # the same (fp32) argument, wherever the value is not lost to that
    # cancellation
    z32 = z[::50].astype(np.float32)
    zt32 = torch.from_numpy(z32.astype(np.float64))
    for kind, ref in ((True, torch.nn.functional.silu(zt32).numpy()),
                      (False, torch.nn.functional.gelu(zt32, approximate="tanh").numpy())):
        for zi, ri in zip(z32, ref):
            if abs(ri) < 1e-6 * max(1.0, abs(float(zi))):
                continue
            got = oracle.act_f32(kind, zi)
            r32 = np.float32(ri)
            assert abs(float(got) - float(r32)) <= np.spacing(np.float32(abs(r32)))


def test_activation_identities():
    assert oracle.gelu_tanh(0.0) == 0.0 and oracle.silu(0.0) == 0.0
    for v in np.linspace(-6, 6, 121):
        # f(z) - f(-z) = z for both tanh-GELU and SiLU
        assert abs(oracle.gelu_tanh(v) - oracle.gelu_tanh(-v) - v) <= 4e-16 * max(1, abs(v))
        assert abs(oracle.silu(v) - oracle.silu(-v) - v) <= 4e-16 * max(1, abs(v))
    assert abs(oracle.gelu_tanh(40.0) - 40.0) < 1e-12 and abs(oracle.gelu_tanh(-40.0)) < 1e-12
    assert abs(oracle.silu(60.0) - 60.0) < 1e-12 and abs(oracle.silu(-60.0)) < 1e-20


def test_weight_quant_scale_and_codes():
    rng = np.random.default_rng(9)
    w = _bf16(rng.standard_normal((64, 128)) * 0.02)
    codes, s = oracle.quant_tensor(w)
    wf = oracle.bf16_to_f32(w)
    amax = np.float32(np.max(np.abs(wf)))
    assert s == np.float32(amax / np.float32(448.0))
    inv = np.float32(np.float32(1.0) / np.float32(s))
    assert np.array_equal(codes, oracle.e4m3_encode((wf * inv).astype(np.float32)))
    # the largest magnitude lands on (or next to) the top code
    assert np.max(np.abs(oracle.e4m3_decode(codes))) >= 416
    # all-zero tensor: scale 1, codes zero
    z = np.zeros((4, 4), np.uint16)
    cz, sz = oracle.quant_tensor(z)
    assert sz == 1.0 and not cz.any()
