"""GPU parity of the attention-input path (K1 + fused QKV projection + split +
rotary embedding) against the CPU oracle, through the C ABI (include/frt_qkv.h).

Checks: weight codes and scale bit-exact; the device rotary table against the
oracle's (fp64 on both sides, each value rounded once to fp32: equal except
where the two fp64 results straddle an fp32 rounding boundary); the
calibration scale; then, with the oracle's table and scale installed,
R' bit-exact, XQ adjacent-code mismatches at <= 1e-4, and Q, K, V within the
block tolerance (max |d| / max |ref| <= 2e-2, cosine >= 0.999) with the
fraction of bit-identical values reported; graph replay equals the eager
forward bit for bit.  Small shapes cover the GEMV (1..4 row tiles, 4/8/16
waves) and the LDS-DMA GEMM, the norm variants, and the three named
workloads run at full size (rows sampled for M=788).
"""
import time

import numpy as np
import pytest
import torch

import oracle
from realtime_transformer_amd import _abi, datagen
from realtime_transformer_amd.configs import QKV_CONFIGS, QkvConfig
from realtime_transformer_amd.plan import QkvPlan, to_np_u16, to_np_u8

from _ffn_case import CODE_RATE, check_codes, check_y, code_stats, log

pytestmark = pytest.mark.gpu

TABLE_MISMATCH_RATE = 1e-5


def run_qkv_case(cfg: QkvConfig, rows=None, flags: int = 0, nbatch: int = 4):
    t0 = time.time()
    M, H = cfg.M, cfg.H
    rows = np.arange(M) if rows is None else np.asarray(sorted(rows))
    log("[qkv %s] M=%d H=%d heads %d/%d x %d flags=%d rows=%d" % (cfg.name, M, H, cfg.nq, cfg.nkv, cfg.hd, flags,
                                                                   len(rows)))
    norm_fuse = bool(flags & _abi.FRT_FLAG_NORM_FUSE)
    ada = bool(flags & _abi.FRT_FLAG_ADA_NORM)
    plan = QkvPlan(M, H, cfg.nq, cfg.nkv, cfg.hd, cfg.max_pos, cfg.eps, cfg.rope_base, flags=flags)
    try:
        wq, wk, wv, wn = datagen.qkv_weights(cfg)
        mod = datagen.modulation(cfg, 0) if ada else None
        plan.load(wq, wk, wv, wn)
        if ada:
            plan.set_modulation(*mod)
        qw = oracle.QkvWeights.quantize(wq, wk, wv, wn, cfg.hd, norm_fuse=norm_fuse, mod=mod)
        got = plan.export_codes()
        nbad = int(np.count_nonzero(got != qw.codes))
        assert nbad == 0, "fused QKV codes: %d mismatches" % nbad
        assert plan.scales()[1] == np.float32(qw.s_w), "weight scale %r vs %r" % (plan.scales()[1], qw.s_w)

        # rotary table
        t_orc = oracle.rope_table(cfg.max_pos, cfg.hd, cfg.rope_base)
        t_gpu = plan.rope().cpu().numpy()
        diff = t_gpu.view(np.int32).astype(np.int64) - t_orc.view(np.int32).astype(np.int64)
        nt = int(np.count_nonzero(diff))
        assert np.abs(diff).max() <= 1, "rotary table differs by more than one fp32 step"
        assert nt <= TABLE_MISMATCH_RATE * diff.size, "rotary table: %d of %d values differ" % (nt, diff.size)
        with torch.cuda.stream(plan.stream):
            plan.rope().copy_(torch.from_numpy(t_orc).to(plan.device))
        plan.sync()

        # calibration (measurement pass) against the oracle's
        cal = datagen.calib_batches(cfg, nbatch)
        plan.calibrate(cal)
        s_x_orc = oracle.qkv_calibrate(cal, qw, cfg.eps)
        rel = abs(float(plan.scales()[0]) / s_x_orc - 1)
        assert rel <= 1e-4, "calibration scale differs by %.3g" % rel
        plan.set_act_scale(s_x_orc)

        r0, y0 = datagen.eval_inputs(cfg)
        pos = datagen.positions(cfg)
        plan.set_inputs(r0, y0, pos)
        plan.capture()
        plan.replay()
        plan.sync()
        outs_graph = [to_np_u16(t) for t in (plan.q(), plan.k(), plan.v())]
        plan.forward()
        plan.sync()
        for a, b, nm in zip(outs_graph, (plan.q(), plan.k(), plan.v()), "QKV"):
            assert np.array_equal(a, to_np_u16(b)), "graph replay and eager forward differ in %s" % nm
        idx = torch.as_tensor(rows, device=plan.device)
        r_g = to_np_u16(plan.r_out()[idx])
        xq_g = to_np_u8(plan.xq()[idx])
        q_g, k_g, v_g = (o[rows] for o in outs_graph)

        r_o, xq_o, q_o, k_o, v_o = oracle.qkv_block(r0[rows], None if y0 is None else y0[rows], qw, cfg.eps, s_x_orc,
                                                    pos[rows], t_orc)
        nb = int(np.count_nonzero(r_g != r_o))
        assert nb == 0, "R': %d bf16 mismatches" % nb
        xs = code_stats(xq_g, xq_o)
        check_codes("XQ", xs)
        res = {}
        for nm, g, o in (("Q", q_g, q_o), ("K", k_g, k_o), ("V", v_g, v_o)):
            mr, cs = check_y(nm, g, o)
            res[nm] = (mr, cs, float(np.mean(g == o)))
        log("[qkv %s] codes/scale exact, table %d/%d differ, XQ %d/%d, %s (%.1fs)" % (
            cfg.name, nt, diff.size, xs.mismatches, xs.n,
            ", ".join("%s max rel %.3g cos %.6f exact %.4f" % (k, *v) for k, v in res.items()), time.time() - t0))
        return res
    finally:
        plan.close()


SMALL = [
    # (index, M, H, nq, nkv, hd, pos0, max_pos, base)
    (121, 1, 256, 2, 1, 64, 5, 64, 10000.0),
    (122, 5, 384, 4, 2, 32, 0, 16, 10000.0),
    (123, 33, 256, 2, 2, 128, 100, 200, 1e6),
    (124, 64, 512, 4, 1, 64, 7, 100, 10000.0),
    (125, 16, 1024, 8, 1, 256, 788, 1024, 10000.0),  # 16 waves
    (126, 100, 256, 4, 2, 64, 3, 128, 10000.0),       # LDS-DMA GEMM, one row tile
    (127, 300, 384, 2, 1, 256, 0, 300, 10000.0),      # LDS-DMA GEMM, ragged row tiles
    (128, 1, 1024, 4, 2, 64, 9, 32, 10000.0),         # one K block per wave
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: "M%d_H%d_%dq%dkv_hd%d" % s[1:6])
def test_qkv_small(spec):
    idx, M, H, nq, nkv, hd, pos0, max_pos, base = spec
    run_qkv_case(QkvConfig(idx, "qkv_small_%d" % idx, M, H, nq, nkv, hd, pos0, max_pos, base))


@pytest.mark.parametrize("spec", [SMALL[1], SMALL[5]], ids=lambda s: "M%d" % s[1])
def test_qkv_small_norm_fuse(spec):
    idx, M, H, nq, nkv, hd, pos0, max_pos, base = spec
    run_qkv_case(QkvConfig(idx, "qkv_normfuse_%d" % idx, M, H, nq, nkv, hd, pos0, max_pos, base),
                 flags=_abi.FRT_FLAG_NORM_FUSE)


@pytest.mark.parametrize("spec", [SMALL[2], SMALL[6]], ids=lambda s: "M%d" % s[1])
def test_qkv_small_ada_norm(spec):
    idx, M, H, nq, nkv, hd, pos0, max_pos, base = spec
    run_qkv_case(QkvConfig(idx, "qkv_ada_%d" % idx, M, H, nq, nkv, hd, pos0, max_pos, base),
                 flags=_abi.FRT_FLAG_ADA_NORM)


@pytest.mark.parametrize("spec", [SMALL[4], SMALL[7]], ids=lambda s: "M%d_H%d" % (s[1], s[2]))
def test_qkv_small_split_norm(spec, monkeypatch):
    # M <= 16 with the norm split (opt-in): slice sums in k_add_sumsq, the
    # quantisation of each wave's K blocks in the QKV GEMV
    monkeypatch.setenv("FRT_QKV_NORM_SPLIT", "1")
    idx, M, H, nq, nkv, hd, pos0, max_pos, base = spec
    run_qkv_case(QkvConfig(idx, "qkv_splitnorm_%d" % idx, M, H, nq, nkv, hd, pos0, max_pos, base))


GEMV_LAUNCH = [
    # nine K blocks: 2 or 3 per wave at 4 waves, 1 or 2 at 8, none for some at 16
    (129, 3, 1152, 4, 2, 64, 11, 64, 10000.0),
    (130, 40, 1152, 2, 1, 128, 0, 64, 1e6),  # three row tiles (16 waves taken as 8)
]


QKV_GEMV_MODES = {"octets": {"FRT_QKV_OCT": "1"},
                  "pairs": {"FRT_QKV_OCT": "0", "FRT_QKV_GEMV_PIPE": "1"},
                  "pairs_unpipelined": {"FRT_QKV_OCT": "0", "FRT_QKV_GEMV_PIPE": "0"}}


@pytest.mark.parametrize("mode", list(QKV_GEMV_MODES))
@pytest.mark.parametrize("waves", ["4", "8", "16"])
@pytest.mark.parametrize("spec", GEMV_LAUNCH, ids=lambda s: "M%d_H%d" % (s[1], s[2]))
def test_qkv_gemv_launch_variants(spec, waves, mode, monkeypatch):
    # the decode GEMV under each wave count: over the octet-ordered weight
    # (one 16-row group per workgroup, the default), or over pairs of groups
    # with and without the two-stage K-block pipeline
    monkeypatch.setenv("FRT_QKV_GEMV_WAVES", waves)
    for k, v in QKV_GEMV_MODES[mode].items():
        monkeypatch.setenv(k, v)
    idx, M, H, nq, nkv, hd, pos0, max_pos, base = spec
    run_qkv_case(QkvConfig(idx, "qkv_gemv_%d_w%s_%s" % (idx, waves, mode), M, H, nq, nkv, hd, pos0, max_pos,
                           base))


def test_qkv_llm_decode_m1_split_norm(monkeypatch):
    monkeypatch.setenv("FRT_QKV_NORM_SPLIT", "1")
    run_qkv_case(QKV_CONFIGS["qkv_llm_decode_m1"])


def test_qkv_action_expert_m50():
    run_qkv_case(QKV_CONFIGS["qkv_action_expert_m50"])


def test_qkv_llm_decode_m1():
    run_qkv_case(QKV_CONFIGS["qkv_llm_decode_m1"])


@pytest.mark.timeout(600)
def test_qkv_vlm_prefix_m788():
    cfg = QKV_CONFIGS["qkv_vlm_prefix_m788"]
    rng = np.random.default_rng(41)
    rows = sorted(set(range(768, 788)) | set(rng.choice(768, 44, replace=False).tolist()))
    run_qkv_case(cfg, rows=rows)


def test_positions_outside_the_table_are_rejected():
    plan = QkvPlan(2, 256, 2, 1, 64, 8)
    try:
        with pytest.raises(_abi.FrtError) as e:
            _abi.frt_qkv_set_positions(plan.plan, np.array([3, 8], np.int32), plan.s)
        assert e.value.status == _abi.FRT_ERR_INVALID_ARG
    finally:
        plan.close()
