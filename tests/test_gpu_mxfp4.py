"""GPU parity of the MXFP4 FFN variant (FRT_FLAG_MXFP4) against the CPU
oracle, through the C ABI.

Checks: packed weight codes and E8M0 exponents equal the oracle's bit for bit
(with and without the AWQ pre-scale); graph replay equals the eager forward;
teacher-forced per block (the oracle's state entering layer l written into
the slots): R' bit-exact, the XQ codes and exponents bit-exact (the same fp32
arithmetic decides them on both sides), HQ codes/exponents at most 1e-4 of
the blocks differing (the GPU sums the products in fp32 in its own order, so
an h value sitting on a rounding or exponent boundary may fall the other
way), Y within the block tolerance (max |d| / max |ref| <= 2e-2, cosine >=
0.999); the free-running chain's Z at cosine >= 0.999 against the oracle's
for chains of at most two layers (reported for deeper ones).
"""
import time

import numpy as np
import pytest
import torch

import oracle
from realtime_transformer_amd import _abi, datagen
from realtime_transformer_amd.configs import CONFIGS, FFNConfig, ACT_GEGLU_TANH, ACT_SWIGLU, ACT_GELU_TANH
from realtime_transformer_amd.plan import FFNPlan, to_np_u16, to_np_u8

from _ffn_case import check_y, log, y_metrics

pytestmark = pytest.mark.gpu

HQ_BLOCK_RATE = 1e-4
MIN_COS = 0.999


def _blocks_differ(codes_g, exps_g, codes_o, exps_o):
    """Number of 32-blocks (per row) whose exponent or any code differs."""
    M, nb = exps_o.shape
    cd = (codes_g != codes_o).reshape(M, nb, 16).any(axis=2)
    return int(np.count_nonzero(cd | (exps_g != exps_o))), M * nb


def _teacher_forced_block(plan, l, r, y, lw, cfg, idx, rows):
    """Write (r, y) into slot l, run layer l alone, compare with the oracle's block."""
    with torch.cuda.stream(plan.stream):
        plan.r_slot(l).index_copy_(0, idx, torch.from_numpy(r.view(np.int16)).to(plan.device))
        if y is None:
            plan.y_slot(l).index_fill_(0, idx, 0)
        else:
            plan.y_slot(l).index_copy_(0, idx, torch.from_numpy(y.view(np.int16)).to(plan.device))
    plan.sync()
    plan.forward_range(l, l + 1)
    plan.sync()
    r_o, xq_o, hq_o, y_o = oracle.block_mxfp4(r, y, lw, cfg.act, cfg.eps)
    r_g = to_np_u16(plan.r_slot(l + 1)[idx])
    assert np.array_equal(r_g, r_o), "layer %d residual differs" % l
    xc, xe = (to_np_u8(t[idx]) for t in plan.xq_mx(l))
    hc, he = (to_np_u8(t[idx]) for t in plan.hq_mx(l))
    a, na = _blocks_differ(xc, xe, *xq_o)
    assert a == 0, "layer %d XQ: %d of %d blocks differ" % (l, a, na)
    b, nb = _blocks_differ(hc, he, *hq_o)
    mr, cs = check_y("layer %d Y" % l, to_np_u16(plan.y_slot(l + 1)[idx]), y_o)
    return a, na, b, nb, mr, cs


def run_mx_case(cfg: FFNConfig, awq: bool = False, flags: int = 0, rows=None, check_layers=None,
                chain: bool = True):
    """chain: the oracle runs the whole chain, its Z is compared with the
    graph's and every checked layer is teacher-forced with the oracle's own
    state entering it (gated at cosine >= 0.999 only for chains of at most
    two layers: deeper random-weight chains amplify summation-order
    differences, reported then).  chain=False: only the checked layers are
    quantised by the oracle and each is compared on fresh seeded (r, y)."""
    t0 = time.time()
    flags |= _abi.FRT_FLAG_MXFP4
    M, H, I, L, act = cfg.M, cfg.H, cfg.I, cfg.L, cfg.act
    rows = np.arange(M) if rows is None else np.asarray(sorted(rows))
    layers = list(range(L)) if check_layers is None else list(check_layers)
    ada = bool(flags & _abi.FRT_FLAG_ADA_NORM)
    log("[mx %s] M=%d H=%d I=%d L=%d act=%d awq=%s flags=%d chain=%s" % (cfg.name, M, H, I, L, act, awq, flags, chain))
    plan = FFNPlan(M, H, I, L, act, cfg.eps, flags=flags)
    try:
        lws = {}
        for l in range(L):
            wg, wu, wd, wn = datagen.layer_weights(cfg, l)
            s = datagen.awq_scales(cfg, l) if awq else None
            mod = datagen.modulation(cfg, l) if ada else None
            if awq:
                plan.set_awq(l, s)
            plan.load_layer(l, wg, wu, wd, wn)
            if ada:
                plan.set_modulation(l, *mod)
            if not chain and l not in layers:
                continue
            lw = oracle.MxLayerWeights.quantize(wg, wu, wd, wn, awq=s, mod=mod)
            for which, ref in ((0, lw.g), (1, lw.u), (2, lw.d)):
                if ref is None:
                    continue
                c, e = plan.export_mx(l, which)
                assert np.array_equal(c, ref[0]), "layer %d tensor %d: %d code bytes differ" % (
                    l, which, int(np.count_nonzero(c != ref[0])))
                assert np.array_equal(e, ref[1]), "layer %d tensor %d: %d exponents differ" % (
                    l, which, int(np.count_nonzero(e != ref[1])))
            lws[l] = lw
            if L > 8 and (l % 8 == 7 or l == L - 1):
                log("[mx %s] layers 0..%d loaded (%.1fs)" % (cfg.name, l, time.time() - t0))
        log("[mx %s] weights bit-exact (%.1fs)" % (cfg.name, time.time() - t0))

        r0, y0 = datagen.eval_inputs(cfg)
        plan.set_inputs(r0, y0)
        plan.capture()
        plan.replay()
        plan.sync()
        z_graph = to_np_u16(plan.z())
        plan.forward()
        plan.sync()
        assert np.array_equal(to_np_u16(plan.z()), z_graph), "eager forward differs from graph replay"
        orc = None
        if chain:
            orc = oracle.run_chain_mxfp4((lambda l=l: lws[l] for l in range(L)), act, cfg.eps, r0[rows],
                                         None if y0 is None else y0[rows])
            z_rel, z_cos = y_metrics(z_graph[rows], oracle.final_hidden(orc.r[L], orc.y[L]))
            log("[mx %s] graph == eager; chain Z cos %.6f max rel %.3g" % (cfg.name, z_cos, z_rel))
            if L <= 2:
                assert z_cos >= MIN_COS, "chain Z cosine %.6f" % z_cos

        idx = torch.as_tensor(rows, device=plan.device)
        nx = nh = nxt = nht = 0
        worst_rel, worst_cos = 0.0, 1.0
        for l in layers:
            if chain:
                r, y = orc.r[l], orc.y[l]
            else:
                r = datagen.residual(cfg, 7000 + 10 * cfg.index + l)[rows]
                y = datagen.normal_bf16(7500 + 10 * cfg.index + l, (cfg.M, cfg.H))[rows]
            a, na, b, nb, mr, cs = _teacher_forced_block(plan, l, r, y, lws[l], cfg, idx, rows)
            nx, nxt, nh, nht = nx + a, nxt + na, nh + b, nht + nb
            worst_rel, worst_cos = max(worst_rel, mr), min(worst_cos, cs)
        assert nh <= HQ_BLOCK_RATE * nht, "HQ: %d of %d blocks differ" % (nh, nht)
        log("[mx %s] per-block: XQ %d/%d blocks, HQ %d/%d blocks differ; Y max rel %.3g min cos %.6f (%.1fs)" % (
            cfg.name, nx, nxt, nh, nht, worst_rel, worst_cos, time.time() - t0))
    finally:
        plan.close()


SMALL = [
    # (index, M, H, I, L, act)
    (131, 1, 512, 1024, 2, ACT_SWIGLU),
    (132, 7, 512, 2048, 2, ACT_GEGLU_TANH),
    (133, 16, 1024, 512, 2, ACT_GELU_TANH),
    (134, 33, 512, 1536, 2, ACT_SWIGLU),
    (135, 64, 1024, 1024, 2, ACT_GEGLU_TANH),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: "M%d_H%d_I%d_act%d" % (s[1], s[2], s[3], s[5]))
def test_mxfp4_small(spec):
    idx, M, H, I, L, act = spec
    run_mx_case(FFNConfig(idx, "mx_small_%d" % idx, M, H, I, L, act))


@pytest.mark.parametrize("spec", [SMALL[0], SMALL[3]], ids=lambda s: "M%d" % s[1])
def test_mxfp4_small_awq(spec):
    idx, M, H, I, L, act = spec
    run_mx_case(FFNConfig(idx, "mx_awq_%d" % idx, M, H, I, L, act), awq=True)


@pytest.mark.parametrize("spec", [SMALL[0], SMALL[2]], ids=lambda s: "M%d" % s[1])
def test_mxfp4_small_one_kernel_norm(spec, monkeypatch):
    # M <= 16 with the whole norm in one kernel (by default it is split: slice
    # sums in k_add_sumsq, quantisation in the gate/up GEMV)
    monkeypatch.setenv("FRT_NORM_SPLIT", "0")
    idx, M, H, I, L, act = spec
    run_mx_case(FFNConfig(idx, "mx_onenorm_%d" % idx, M, H, I, L, act), awq=True)


def test_mxfp4_small_split_norm_slices():
    # the split norm with 16 slice sums per row (H = 8192)
    run_mx_case(FFNConfig(136, "mx_splitnorm_136", 1, 8192, 512, 2, ACT_GEGLU_TANH), awq=True)


def test_mxfp4_small_ada_norm():
    idx, M, H, I, L, act = SMALL[1]
    run_mx_case(FFNConfig(idx, "mx_ada_%d" % idx, M, H, I, L, act), flags=_abi.FRT_FLAG_ADA_NORM)


# the whole-column down GEMV (M <= 4 on the split norm: the down matrix in
# the column-quad order, the next layer's R' and slice sums formed in its
# epilogue, no norm kernel between layers): uneven step shares over the
# waves, a single step on a single wave, every activation, rows 1..4, and
# the gate/up prologue's slice-sum loads filled to their limit (M = 4,
# H = 2048 on four waves)
MX_QUAD = [
    (160, 1, 512, 2560, 3, ACT_SWIGLU),
    (161, 2, 1024, 1024, 2, ACT_GEGLU_TANH),
    (162, 3, 512, 512, 2, ACT_GELU_TANH),
    (163, 4, 2048, 1536, 2, ACT_SWIGLU),
]


def _mx_path(M, H, I, L, act):
    plan = FFNPlan(M, H, I, L, act, 1e-6, flags=_abi.FRT_FLAG_MXFP4)
    try:
        return plan.path()
    finally:
        plan.close()


@pytest.mark.parametrize("spec", MX_QUAD, ids=lambda s: "M%d_H%d_I%d_act%d" % (s[1], s[2], s[3], s[5]))
def test_mxfp4_small_down_whole_column(spec):
    idx, M, H, I, L, act = spec
    assert _mx_path(M, H, I, L, act) & _abi.FRT_PATH_DOWN_WHOLE_COLUMN
    run_mx_case(FFNConfig(idx, "mx_quad_%d" % idx, M, H, I, L, act), awq=True)


@pytest.mark.parametrize("spec", [MX_QUAD[0], MX_QUAD[3]], ids=lambda s: "M%d" % s[1])
def test_mxfp4_small_down_split_k(spec, monkeypatch):
    # FRT_DOWN_QUAD=0: the down GEMV on 16-column workgroups (K split in two
    # at I = 2560, whole at I = 1536) and the slice-sum kernel
    monkeypatch.setenv("FRT_DOWN_QUAD", "0")
    idx, M, H, I, L, act = spec
    path = _mx_path(M, H, I, L, act)
    assert not path & _abi.FRT_PATH_DOWN_WHOLE_COLUMN
    assert bool(path & _abi.FRT_PATH_DOWN_SPLIT_K) == (I == 2560)
    run_mx_case(FFNConfig(idx, "mx_splitk_%d" % idx, M, H, I, L, act), awq=True)


# the block-scaled prefill GEMM (M > 64): one and several 128-row tiles,
# ragged tails, all three activations, the K-split down GEMM
MM = [
    (137, 65, 512, 1024, 2, ACT_SWIGLU),
    (138, 100, 1024, 512, 2, ACT_GELU_TANH),
    (139, 300, 512, 2048, 2, ACT_GEGLU_TANH),
]


@pytest.mark.parametrize("spec", MM, ids=lambda s: "M%d_H%d_I%d_act%d" % (s[1], s[2], s[3], s[5]))
def test_mxfp4_prefill_small(spec):
    idx, M, H, I, L, act = spec
    run_mx_case(FFNConfig(idx, "mx_mm_%d" % idx, M, H, I, L, act))


def test_mxfp4_prefill_awq():
    run_mx_case(FFNConfig(140, "mx_mm_awq", 129, 1024, 1536, 2, ACT_SWIGLU), awq=True)


@pytest.mark.timeout(900)
def test_mxfp4_vlm_prefix_m788_full_size():
    # the pages' 4-bit encoder FFN shape: 18 layers, 768 image + 20 text rows
    cfg = CONFIGS[3]
    rng = np.random.default_rng(37)
    rows = sorted(set(range(768, 788)) | set(rng.choice(768, 44, replace=False).tolist()))
    run_mx_case(cfg, awq=True, rows=rows)


def test_mxfp4_action_expert_m50_chain():
    run_mx_case(CONFIGS[2], awq=True)


@pytest.mark.timeout(900)
def test_mxfp4_llm_decode_m1_full_size():
    # all 64 layers on the GPU (graph == eager); the oracle checks a spread of
    # layers on fresh seeded inputs
    run_mx_case(CONFIGS[4], awq=True, check_layers=[0, 1, 21, 42, 63], chain=False)


# E2M1 decision points (between neighbouring magnitudes) and the grid itself,
# in units of the block scale
_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _edge_weights(rows, cols, seed):
    """bf16 bits [rows, cols] built so that every 32-block tests the encoder at
    its boundaries: one value of magnitude 6 * 2^k or 7.5 * 2^k fixes the
    block exponent at 127 + k (clamped to 0 for the smallest k), the other 31
    are drawn from the midpoints, one bf16 step below and above each, the grid,
    values past 6 (saturating), zeros of both signs and bf16 subnormals, each
    times 2^k with a random sign.  A few blocks are all +0 or all -0."""
    rng = np.random.default_rng(seed)
    mid = datagen.to_bf16_bits(np.array(_E2M1_MIDPOINTS, np.float32)).astype(np.int64)
    pool_bits = np.concatenate([mid, mid - 1, mid + 1])
    pool = np.concatenate([
        pool_bits.astype(np.uint16).view(np.uint16).astype(np.uint32) << 16,
        (datagen.to_bf16_bits(np.array(_E2M1_GRID + (6.5, 7.0, 7.5), np.float32)).astype(np.uint32) << 16),
    ]).view(np.float32)
    nb = cols // 32
    out = np.empty((rows, cols), np.float32)
    ks = rng.integers(-40, 12, size=(rows, nb))
    low = rng.random((rows, nb)) < 0.05  # the exponent clamp region
    ks[low] = rng.integers(-133, -122, size=int(low.sum()))
    for r in range(rows):
        for b in range(nb):
            k = int(ks[r, b])
            v = rng.choice(pool, 32) * rng.choice(np.array([-1.0, 1.0], np.float32), 32)
            v[rng.integers(32)] = rng.choice(np.array([6.0, 7.5, -6.0, -7.5], np.float32))
            out[r, b * 32:(b + 1) * 32] = np.ldexp(v.astype(np.float64), k).astype(np.float32)
    bits = datagen.to_bf16_bits(out)
    sub = rng.random((rows, cols)) < 0.02  # bf16 subnormals (both signs)
    bits[sub] = (rng.integers(1, 128, size=int(sub.sum())) | (rng.integers(0, 2, size=int(sub.sum())) << 15)).astype(
        np.uint16)
    bits[0, :32] = 0x0000
    bits[1, :32] = 0x8000
    return bits


def test_mxfp4_weight_codes_on_rounding_boundaries():
    """The device encoder (codes and block exponents of the packed weights,
    both exponent layouts) against the oracle's on values placed on and next to
    every E2M1 rounding boundary, in blocks whose exponent spans the clamp."""
    for M in (1, 100):  # GEMV and prefill exponent layouts
        cfg = FFNConfig(141, "mx_edges", M, 512, 512, 1, ACT_SWIGLU)
        wg, wu, wd = (_edge_weights(r, c, 90 + i) for i, (r, c) in enumerate(((512, 512), (512, 512), (512, 512))))
        wn = datagen.layer_weights(cfg, 0)[3]
        plan = FFNPlan(cfg.M, cfg.H, cfg.I, cfg.L, cfg.act, cfg.eps, flags=_abi.FRT_FLAG_MXFP4)
        try:
            plan.load_layer(0, wg, wu, wd, wn)
            lw = oracle.MxLayerWeights.quantize(wg, wu, wd, wn)
            for which, ref in ((0, lw.g), (1, lw.u), (2, lw.d)):
                c, e = plan.export_mx(0, which)
                assert np.array_equal(e, ref[1]), "M=%d tensor %d: %d exponents differ" % (
                    M, which, int(np.count_nonzero(e != ref[1])))
                assert np.array_equal(c, ref[0]), "M=%d tensor %d: %d code bytes differ" % (
                    M, which, int(np.count_nonzero(c != ref[0])))
            log("[mx edges M=%d] codes and exponents bit-exact; exponents span %d..%d" % (
                M, int(lw.u[1].min()), int(lw.u[1].max())))
        finally:
            plan.close()


def test_mxfp4_rejects_calibration_and_fp8_exports():
    cfg = FFNConfig(136, "mx_api", 2, 512, 512, 1, ACT_SWIGLU)
    plan = FFNPlan(cfg.M, cfg.H, cfg.I, cfg.L, cfg.act, cfg.eps, flags=_abi.FRT_FLAG_MXFP4)
    try:
        wg, wu, wd, wn = datagen.layer_weights(cfg, 0)
        plan.load_layer(0, wg, wu, wd, wn)
        with pytest.raises(_abi.FrtError) as e:
            plan.calibrate(datagen.calib_batches(cfg, 1))
        assert e.value.status == _abi.FRT_ERR_UNSUPPORTED
        with pytest.raises(_abi.FrtError) as e:
            plan.export_codes(0, 1)
        assert e.value.status == _abi.FRT_ERR_STATE
        bad = np.zeros(cfg.H, np.uint16)  # scale 0 is rejected
        with pytest.raises(_abi.FrtError) as e:
            plan.set_awq(0, bad)
        assert e.value.status == _abi.FRT_ERR_INVALID_ARG
    finally:
        plan.close()
