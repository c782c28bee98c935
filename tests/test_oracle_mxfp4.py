"""Pins of the oracle's MXFP4 variant (itsolotime article section 7.2: the
4-bit encoder FFN with AWQ pre-scale; OCP Microscaling MXFP4 as the format):
the E2M1 value table, the rounding ties and saturation, the E8M0 block
exponent, nibble packing, the exact block-scaled GEMM against rational
arithmetic, and the AWQ orientation through a power-of-two invariance."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_ocp_values.txt")


def _table():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    return {int(c, 16): float(v) for c, v in rows}


def test_decode_matches_the_ocp_table():
    t = _table()
    assert len(t) == 16
    got = oracle.e2m1_decode(np.arange(16))
    for c, v in t.items():
        assert got[c] == v and np.signbit(got[c]) == np.signbit(v), c


def test_encode_round_trips_every_code():
    vals = oracle.e2m1_decode(np.arange(16))
    assert np.array_equal(oracle.e2m1_encode(vals), np.arange(16, dtype=np.uint8))


@pytest.mark.parametrize("v,expect", [
    (0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0), (3.5, 4.0), (5.0, 4.0),   # ties: even mantissa
    (0.2500001, 0.5), (0.7499999, 0.5), (4.999, 4.0), (5.001, 6.0),                           # either side
    (6.0, 6.0), (6.9, 6.0), (1e30, 6.0), (-7.5, -6.0), (-0.1, -0.0), (0.0, 0.0)])              # saturation, sign
def test_encode_rounding(v, expect):
    c = oracle.e2m1_encode([v])[0]
    d = oracle.e2m1_decode([c])[0]
    assert d == expect and np.signbit(d) == np.signbit(expect), (v, c, d)


def test_encode_is_monotone_and_nearest():
    t = sorted(set(abs(v) for v in _table().values()))
    x = np.linspace(0, 8, 20001)
    d = oracle.e2m1_decode(oracle.e2m1_encode(x))
    assert np.all(np.diff(d) >= 0)
    dist = np.abs(d - x)
    best = np.min(np.abs(np.asarray(t)[None, :] - x[:, None]), axis=1)
    assert np.all(dist == best)


@pytest.mark.parametrize("amax,e", [
    (6.0, 127), (4.0, 127), (7.99, 127), (1.0, 125), (0.75, 124), (3.0, 126),
    (0.0, 0), (2.0 ** -140, 0), (2.0 ** 200, 254)])
def test_block_exponent(amax, e):
    assert oracle.mx_scale_exp(amax) == e


def test_block_quantisation_packing_and_clipping():
    v = np.zeros((1, 64), np.float32)
    v[0, 0] = 3.0            # block 0: amax 3 -> e = 126 (X = 0.5): 3 / 0.5 = 6
    v[0, 1] = -0.5           # -0.5 / 0.5 = -1 -> code 0xA in the high nibble
    v[0, 32:64] = 0.0        # block 1: all zero -> e = 0, codes 0
    v[0, 33] = 0.0
    codes, scales = oracle.mxfp4_quant_rows(v)
    assert scales.tolist() == [[126, 0]]
    assert codes[0, 0] == 0xA7          # element 0 low nibble (6.0 = 0x7), element 1 high nibble
    assert not np.any(codes[0, 16:])
    w = np.zeros((1, 32), np.float32)
    w[0, :] = 7.0                       # amax 7: X = 1, values clip to 6 (OCP rule)
    c2, s2 = oracle.mxfp4_quant_rows(w)
    assert s2[0, 0] == 127 and np.all(c2 == 0x77)


def test_power_of_two_scaling_moves_only_the_exponent():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((3, 96)).astype(np.float32)
    c1, s1 = oracle.mxfp4_quant_rows(v)
    c2, s2 = oracle.mxfp4_quant_rows(v * np.float32(2.0 ** 5))
    assert np.array_equal(c1, c2) and np.array_equal(s2.astype(int), s1.astype(int) + 5)


def _dequant(codes, scales):
    vals = oracle.e2m1_decode(np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1))
    return [[Fraction(float(vals[r, k])) * Fraction(2) ** (int(scales[r, k // 32]) - 127)
             for k in range(vals.shape[1])] for r in range(vals.shape[0])]


def _f32_nearest(fr: Fraction) -> np.float32:
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    dist = [abs(Fraction(float(c)) - fr) for c in cands]
    best = min(dist)
    ties = [c for c, d in zip(cands, dist) if d == best]
    return min(ties, key=lambda c: int(np.float32(c).view(np.uint32)) & 1)


def test_gemm_is_the_exact_sum_rounded_once():
    rng = np.random.default_rng(4)
    a = (rng.standard_normal((3, 96)) * np.exp2(rng.integers(-6, 6, (3, 96)))).astype(np.float32)
    b = (rng.standard_normal((5, 96)) * np.exp2(rng.integers(-6, 6, (5, 96)))).astype(np.float32)
    ac, as_ = oracle.mxfp4_quant_rows(a)
    bc, bs = oracle.mxfp4_quant_rows(b)
    out = oracle.mxfp4_gemm(ac, as_, bc, bs)
    A, B = _dequant(ac, as_), _dequant(bc, bs)
    for m in range(3):
        for n in range(5):
            exact = sum(x * y for x, y in zip(A[m], B[n]))
            assert out[m, n] == _f32_nearest(exact), (m, n)
    assert out.shape == (3, 5)  # [M][N]: a transposed operand would give 5 x 3


def test_gemm_refuses_an_inexact_spread():
    a = np.zeros((1, 64), np.float32)
    a[0, 0] = 2.0 ** 60
    a[0, 32] = 2.0 ** -60
    ac, as_ = oracle.mxfp4_quant_rows(a)
    with pytest.raises(ValueError):
        oracle.mxfp4_gemm(ac, as_, ac, as_)


def _bf16(x):
    return oracle.bf16_round(np.asarray(x, np.float32))


def _layer(seed, H, I, gated=True):
    rng = np.random.default_rng(seed)
    wg = _bf16(rng.standard_normal((I, H)) * 0.02) if gated else None
    wu = _bf16(rng.standard_normal((I, H)) * 0.02)
    wd = _bf16(rng.standard_normal((H, I)) * 0.02)
    wn = _bf16(1 + 0.1 * rng.standard_normal(H))
    return wg, wu, wd, wn


def test_awq_by_powers_of_two_changes_nothing():
    # s[k] = 2^j for all k of a 32-block (j varying between blocks): W*s and
    # x/s shift each block's exponent by +j and -j exactly, so every code and
    # output is unchanged; a row-wise or uninverted scale fails
    M, H, I = 4, 128, 256
    wg, wu, wd, wn = _layer(5, H, I)
    rng = np.random.default_rng(6)
    r = _bf16(rng.standard_normal((M, H)))
    s = _bf16(np.repeat(np.exp2(rng.integers(-3, 4, H // 32).astype(np.float32)), 32))
    plain = oracle.block_mxfp4(r, None, oracle.MxLayerWeights.quantize(wg, wu, wd, wn), 0, 1e-6)
    awq = oracle.block_mxfp4(r, None, oracle.MxLayerWeights.quantize(wg, wu, wd, wn, awq=s), 0, 1e-6)
    assert np.array_equal(plain[3], awq[3])
    assert np.array_equal(plain[2][0], awq[2][0]) and np.array_equal(plain[2][1], awq[2][1])
    # a uniform power of two s = 2^k shifts every activation block exponent by -k
    s2 = np.full(H, _bf16([4.0])[0], np.uint16)
    awq2 = oracle.block_mxfp4(r, None, oracle.MxLayerWeights.quantize(wg, wu, wd, wn, awq=s2), 0, 1e-6)
    assert np.array_equal(awq2[1][1].astype(int), plain[1][1].astype(int) - 2)
    assert np.array_equal(awq2[3], plain[3])


def test_block_wiring_and_zero_weights():
    M, H, I = 3, 64, 128
    wg, wu, wd, wn = _layer(7, H, I)
    rng = np.random.default_rng(8)
    r = _bf16(rng.standard_normal((M, H)))
    y = _bf16(rng.standard_normal((M, H)))
    lw = oracle.MxLayerWeights.quantize(wg, wu, wd, wn)
    r_out, (xc, xs), (hc, hs), y_out = oracle.block_mxfp4(r, y, lw, 1, 1e-6)
    r_ref, x, _ = oracle.add_rmsnorm_quant(r, y, wn, 1e-6, 1.0)
    assert np.array_equal(r_out, r_ref)
    c, sc = oracle.mxfp4_quant_rows(x)
    assert np.array_equal(xc, c) and np.array_equal(xs, sc)
    g = oracle.mxfp4_gemm(xc, xs, *lw.g)
    u = oracle.mxfp4_gemm(xc, xs, *lw.u)
    h = np.array([[np.float32(np.float32(oracle.silu(float(gg))) * uu) for gg, uu in zip(gr, ur)]
                  for gr, ur in zip(g, u)], np.float32)
    c, sc = oracle.mxfp4_quant_rows(h)
    assert np.array_equal(hc, c) and np.array_equal(hs, sc)
    d = oracle.mxfp4_gemm(hc, hs, *lw.d)
    assert np.array_equal(y_out, _bf16(d))
    zero = oracle.MxLayerWeights.quantize(np.zeros_like(wg), np.zeros_like(wu), np.zeros_like(wd), wn)
    _, _, _, y0 = oracle.block_mxfp4(r, y, zero, 0, 1e-6)
    assert not np.any(y0 & 0x7FFF)


def test_mxfp4_tracks_the_fp8_block():
    # the 4-bit block stays within a few percent of the E4M3 block's output
    M, H, I = 8, 256, 512
    wg, wu, wd, wn = _layer(9, H, I)
    rng = np.random.default_rng(10)
    r = _bf16(rng.standard_normal((M, H)))
    y4 = oracle.block_mxfp4(r, None, oracle.MxLayerWeights.quantize(wg, wu, wd, wn), 0, 1e-6)[3]
    lw8 = oracle.LayerWeights.quantize(wg, wu, wd, wn)
    _, _, ax, ah = oracle.block_measure(r, None, lw8, 0, 1e-6)
    y8 = oracle.block(r, None, lw8, 0, 1e-6, oracle.scale_from_amax(ax), oracle.scale_from_amax(ah))[3]
    a = oracle.bf16_to_f32(y4).astype(np.float64).ravel()
    b = oracle.bf16_to_f32(y8).astype(np.float64).ravel()
    cos = a @ b / (np.linalg.norm(a) * np.linalg.norm(b))
    assert 0.95 < cos < 1.0
