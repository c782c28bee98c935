"""Pins of the oracle's whole block, chain and calibration.

* an independent transcription of the block in torch float64 with torch's
  own float8/bf16 casts (different code, library conversions) must give the
  same bytes on tiny shapes for all three activations;
* zero weights give Y = 0 and Z = R[0] exactly;
* rows are independent: permuting the rows permutes every output;
* calibration scales equal a brute-force max over the measurement chain;
* the split GEMM + epilogue equals the fused step.
"""
import math

import numpy as np
import pytest
import torch

import oracle

ACTS = [oracle.ACT_GEGLU_TANH, oracle.ACT_SWIGLU, oracle.ACT_GELU_TANH]


def _bf16(x):
    return oracle.bf16_round(np.asarray(x, np.float32))


def _layer(rng, H, I, act, scale=0.02):
    wg = _bf16(rng.standard_normal((I, H)) * scale) if act != oracle.ACT_GELU_TANH else None
    wu = _bf16(rng.standard_normal((I, H)) * scale)
    wd = _bf16(rng.standard_normal((H, I)) * scale)
    wn = _bf16(1.0 + 0.1 * rng.standard_normal(H))
    return wg, wu, wd, wn


def _torch_block(r, y, wg, wu, wd, wn, act, eps, s_x, s_h):
    """Block written with torch ops only (fp64 math, torch float8/bf16 casts)."""
    t = lambda b: torch.from_numpy(oracle.bf16_to_f32(b).astype(np.float32))
    f8 = lambda v: v.clamp(-448, 448).to(torch.float8_e4m3fn)
    def quantw(w):
        wt = t(w)
        amax = wt.abs().max()
        s = (amax / torch.tensor(448.0, dtype=torch.float32)) if amax > 0 else torch.tensor(1.0)
        inv = torch.tensor(1.0, dtype=torch.float32) / s
        return f8(wt * inv), s
    rr = (t(r) + (t(y) if y is not None else 0)).to(torch.bfloat16).to(torch.float32)
    S = (rr.double() ** 2).sum(1, keepdim=True)
    inv_rms = (1.0 / torch.sqrt(S / rr.shape[1] + float(np.float32(eps)))).to(torch.float32)
    x = (rr * inv_rms) * t(wn)
    inv_x = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(s_x, dtype=torch.float32)
    xq = f8(x * inv_x)
    qu, su = quantw(wu)
    qd, sd = quantw(wd)
    a_u = torch.tensor(s_x, dtype=torch.float32) * su
    Au = (xq.double() @ qu.double().T).to(torch.float32)
    u = Au * a_u
    if act == oracle.ACT_GELU_TANH:
        h = torch.nn.functional.gelu(u.double(), approximate="tanh").to(torch.float32)
    else:
        qg, sg = quantw(wg)
        a_g = torch.tensor(s_x, dtype=torch.float32) * sg
        g = (xq.double() @ qg.double().T).to(torch.float32) * a_g
        if act == oracle.ACT_SWIGLU:
            a = torch.nn.functional.silu(g.double()).to(torch.float32)
        else:
            a = torch.nn.functional.gelu(g.double(), approximate="tanh").to(torch.float32)
        h = a * u
    inv_h = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(s_h, dtype=torch.float32)
    hq = f8(h * inv_h)
    a_d = torch.tensor(s_h, dtype=torch.float32) * sd
    Ad = (hq.double() @ qd.double().T).to(torch.float32)
    yo = (Ad * a_d).to(torch.bfloat16)
    as_u8 = lambda v: v.view(torch.uint8).numpy()
    as_u16 = lambda v: v.view(torch.int16).numpy().view(np.uint16)
    return as_u16(rr.to(torch.bfloat16)), as_u8(xq), as_u8(hq), as_u16(yo)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("M,H,I", [(1, 64, 128), (3, 64, 128), (4, 128, 192)])
def test_block_matches_torch_transcription(act, M, H, I):
    rng = np.random.default_rng(M * 100 + H + act)
    r = _bf16(rng.standard_normal((M, H)))
    y = _bf16(rng.standard_normal((M, H)))
    wg, wu, wd, wn = _layer(rng, H, I, act, scale=0.05)
    lw = oracle.LayerWeights.quantize(wg, wu, wd, wn)
    s_x, s_h = 0.011, 0.0023
    got = oracle.block(r, y, lw, act, 1e-6, s_x, s_h)
    ref = _torch_block(r, y, wg, wu, wd, wn, act, 1e-6, s_x, s_h)
    for name, g, e in zip(("r", "xq", "hq", "y"), got, ref):
        assert np.array_equal(g, e), name


def test_zero_weights_pass_residual_through():
    rng = np.random.default_rng(5)
    M, H, I = 3, 64, 128
    r = _bf16(rng.standard_normal((M, H)))
    z = np.zeros((I, H), np.uint16)
    lw = oracle.LayerWeights.quantize(z, z, np.zeros((H, I), np.uint16), _bf16(np.ones(H)))
    res = oracle.calibrate_and_run([lambda: lw, lambda: lw], oracle.ACT_SWIGLU, 1e-6, r, None,
                                   [(r, None)])
    assert np.array_equal(res.r[1], r) and np.array_equal(res.r[2], r)
    assert not res.y[1].any() and not res.y[2].any()
    assert np.array_equal(oracle.final_hidden(res.r[2], res.y[2]), r)


def test_rows_are_independent():
    rng = np.random.default_rng(6)
    M, H, I = 9, 128, 256
    r = _bf16(rng.standard_normal((M, H)))
    y = _bf16(rng.standard_normal((M, H)))
    lw = oracle.LayerWeights.quantize(*_layer(rng, H, I, oracle.ACT_GEGLU_TANH))
    perm = rng.permutation(M)
    a = oracle.block(r, y, lw, oracle.ACT_GEGLU_TANH, 1e-6, 0.01, 0.003)
    b = oracle.block(r[perm], y[perm], lw, oracle.ACT_GEGLU_TANH, 1e-6, 0.01, 0.003)
    for x, xp in zip(a, b):
        assert np.array_equal(x[perm], xp)
    c = oracle.block(r[2:5], y[2:5], lw, oracle.ACT_GEGLU_TANH, 1e-6, 0.01, 0.003)
    for x, xs in zip(a, c):
        assert np.array_equal(x[2:5], xs)


def test_calibration_is_brute_force_max():
    rng = np.random.default_rng(7)
    M, H, I = 5, 64, 128
    lws = [oracle.LayerWeights.quantize(*_layer(rng, H, I, oracle.ACT_SWIGLU)) for _ in range(2)]
    batches = [(_bf16(rng.standard_normal((M, H))), None) for _ in range(3)]
    res = oracle.calibrate_and_run([(lambda lw=lw: lw) for lw in lws], oracle.ACT_SWIGLU, 1e-6,
                                   batches[0][0], None, batches, keep_cal_states=True)
    for l, lw in enumerate(lws):
        ax = ah = 0.0
        for (r, y) in res.cal_states[l]:
            _, x, _ = oracle.add_rmsnorm_quant(r, y, lw.w_norm, 1e-6, 1.0, mod=lw.mod)
            ax = max(ax, float(np.abs(x).max()))
            # h recomputed from the definition with fp64 sums
            dec = lambda c: oracle.e4m3_decode(c)
            g = np.float32(lw.s_g) * (x.astype(np.float64) @ dec(lw.qg).T)
            u = np.float32(lw.s_u) * (x.astype(np.float64) @ dec(lw.qu).T)
            g = g.astype(np.float32)
            u = u.astype(np.float32)
            a = np.array([oracle.act_f32(True, v) for v in g.ravel()], np.float32).reshape(g.shape)
            ah = max(ah, float(np.abs(a * u).max()))
        assert res.amax_x[l] == np.float32(ax)
        assert abs(res.amax_h[l] / ah - 1) < 1e-6
        assert res.s_x[l] == np.float32(np.float32(res.amax_x[l]) / np.float32(448))
        assert np.float32(res.s_h[l]) * np.float32(448) >= np.float32(res.amax_h[l]) * (1 - 1e-7)


@pytest.mark.parametrize("act", ACTS)
def test_split_epilogue_equals_fused_step(act):
    rng = np.random.default_rng(8)
    M, H, I = 4, 128, 256
    wg, wu, wd, wn = _layer(rng, H, I, act)
    lw = oracle.LayerWeights.quantize(wg, wu, wd, wn)
    xq = oracle.e4m3_encode((rng.standard_normal((M, H)) * 50).astype(np.float32))
    h, hq = oracle.gateup(xq, lw.qg, lw.qu, act, 1e-3, 2e-3, 50.0)
    Au = oracle.gemm_e4m3(xq, lw.qu)
    Ag = None if lw.qg is None else oracle.gemm_e4m3(xq, lw.qg)
    h2, hq2 = oracle.gateup_epilogue(Ag, Au, act, 1e-3, 2e-3, 50.0)
    assert np.array_equal(h, h2) and np.array_equal(hq, hq2)
    yd = oracle.down(hq, lw.qd, 1e-4)
    assert np.array_equal(yd, oracle.down_epilogue(oracle.gemm_e4m3(hq, lw.qd), 1e-4))
