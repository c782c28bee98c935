"""Shared GPU-vs-oracle parity procedure for one FFN-chain workload.

Direction of data: seeded inputs (datagen) feed both sides; the oracle runs
its own chain from them; its per-layer states are written INTO the GPU's
slots for the teacher-forced per-block checks.  Nothing read back from the
GPU is ever given to the oracle.

Checks (tolerances from the workload statement; C-19 reading for HQ):
  weights   GPU codes and scales equal the oracle's bit for bit
  calib     GPU activation scales within CAL_RTOL of the oracle's (the GPU
            sums fp32 in its own order, the oracle in fp64)
  per block (teacher-forced, every checked layer):
            R  bit-exact
            XQ every mismatch adjacent and within 1 fp32 ulp of the E4M3
               rounding boundary (its inputs are identical on both sides),
               rate <= 1e-4
            HQ adjacent-code mismatches only, rate <= 1e-4, and each one
               reachable by an fp32 accumulation error of at most
               T_MAX_EXPLAINED units (tests/_hq_explain.py)
            Y  max|d|/max|ref| <= 2e-2 and cosine >= 0.999
  chain     free-running: the GPU's distance from the oracle (1 - cosine of
            Z) against the spread of several valid fp32 summation orders
            (tests/_natural.py)
  graph     replay == eager forward, bit for bit; two replays agree
  saturation every XQ/HQ code finite (no 0x7f/0xff)
"""
from __future__ import annotations

import json
import math
import os
import time
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

import oracle
from realtime_transformer_amd import _abi, datagen
from realtime_transformer_amd.configs import FFNConfig
from realtime_transformer_amd.plan import FFNPlan, to_np_u16, to_np_u8

import _hq_explain
import _natural

CODE_RATE = 1e-4
Y_MAX_REL = 2e-2
MIN_COS = 0.999
# Calibration scales: |s_gpu/s_oracle - 1|.  In the first layer both sides
# see identical inputs and differ only by the GPU's fp32 K-sequential sums
# against the oracle's fp64 sums (~sqrt(K) * 2^-24 relative, 1e-3 worst
# case at K = 16384): CAL_RTOL_FIRST.  Deeper layers measure a chain whose
# bf16 residual and previous output may round the other way in single
# elements (2^-8 = 0.4% of that element) and propagate; amax over the layer
# then moves by up to a few of those steps: CAL_RTOL.
CAL_RTOL_FIRST = 1e-4
CAL_RTOL = 1e-2
# Free-running chain (no teacher forcing): Z must reach cosine >= MIN_COS
# against the oracle's chain, or, where valid implementations themselves
# drift further than that (the 64-layer M=1 chain), the GPU's distance
# (1 - cosine) may be at most DRIFT_FACTOR times the largest distance of the
# valid fp32 summation orders in tests/_natural.py, plus a floor for chains
# too short to drift.  DRIFT_FACTOR: across the five workloads the largest
# of those distances is up to 2.1x the smallest (M=4096: 3.4e-4 to 7.1e-4),
# so an implementation with yet another valid order can sit that far above
# the largest; rounded up to 2.5.
DRIFT_FACTOR = 2.5
DRIFT_FLOOR = 1e-6
NATURAL_DRIFT_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "natural_drift.json")


def stored_natural_drift(cfg: FFNConfig, rows, cal_rows) -> Optional[dict]:
    """Distances of the valid orders for a named workload, stored by
    tests/golden/make_natural_drift.py (the oracle and tests/_natural.py
    only), or None if there is no record for these rows."""
    if not os.path.exists(NATURAL_DRIFT_FILE):
        return None
    rec = json.load(open(NATURAL_DRIFT_FILE)).get(cfg.name)
    if rec is None:
        return None
    want_rows = None if rows is None else [int(r) for r in rows]
    want_cal = None if cal_rows is None else [int(r) for r in cal_rows]
    if rec["rows"] != want_rows or rec["cal_rows"] != want_cal or rec["shape"] != [cfg.M, cfg.H, cfg.I, cfg.L]:
        return None
    return rec["distances"]
# Free-running whole-chain calibration: after tens of layers the measurement
# chains of two valid implementations (fp32 vs fp64 sums) drift apart by a
# few percent in amax; gated only as a sanity bound.  The per-layer check
# below feeds both sides the same states and is gated at CAL_RTOL_FIRST.
CAL_DRIFT_MAX = 0.1


def log(msg: str):
    print(msg, flush=True)


def e4m3_rank(codes: np.ndarray) -> np.ndarray:
    c = codes.astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


@dataclass
class CodeStats:
    n: int
    mismatches: int
    max_rank_diff: int
    near_boundary: int = -1

    @property
    def rate(self) -> float:
        return self.mismatches / max(1, self.n)


def code_stats(gpu: np.ndarray, ref: np.ndarray, pre: Optional[np.ndarray] = None) -> CodeStats:
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    d = np.abs(e4m3_rank(gpu) - e4m3_rank(ref))
    bad = d > 0
    st = CodeStats(int(gpu.size), int(bad.sum()), int(d.max()) if d.size else 0)
    if pre is not None and st.mismatches:
        # mismatches whose oracle pre-rounding value lies within 1 fp32 ulp
        # of the rounding boundary between the two codes
        v = pre[bad].astype(np.float32)
        a = oracle.e4m3_decode(gpu[bad])
        b = oracle.e4m3_decode(ref[bad])
        mid = (a + b) / 2
        ulp = np.spacing(np.abs(v)).astype(np.float64)
        st.near_boundary = int(np.sum(np.abs(v.astype(np.float64) - mid) <= ulp))
    return st


class CodeToleranceMiss(AssertionError):
    """An FP8 byte tolerance (rate, adjacency or boundary rule) is missed."""


def check_codes(name: str, st: CodeStats, boundary_rule: bool = False):
    """Adjacency and rate; with boundary_rule (XQ, whose inputs are identical
    on both sides) every mismatch must also lie within 1 fp32 ulp of the
    rounding boundary between the two codes."""
    if st.max_rank_diff > 1:
        raise CodeToleranceMiss("%s: non-adjacent code mismatch (%d steps)" % (name, st.max_rank_diff))
    if st.rate > CODE_RATE:
        raise CodeToleranceMiss("%s: code mismatch rate %.3g > %g (%d/%d)" % (
            name, st.rate, CODE_RATE, st.mismatches, st.n))
    if boundary_rule and st.mismatches and st.near_boundary != st.mismatches:
        raise CodeToleranceMiss("%s: %d of %d mismatches are not within 1 fp32 ulp of a rounding boundary" % (
            name, st.mismatches - st.near_boundary, st.mismatches))


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return oracle.bf16_to_f32(bits).astype(np.float64)


def y_metrics(gpu_bits: np.ndarray, ref_bits: np.ndarray):
    g = bf16_f64(gpu_bits).ravel()
    r = bf16_f64(ref_bits).ravel()
    denom = np.max(np.abs(r))
    max_rel = float(np.max(np.abs(g - r)) / denom) if denom > 0 else float(np.max(np.abs(g)))
    ng, nr = np.linalg.norm(g), np.linalg.norm(r)
    cos = float(g @ r / (ng * nr)) if ng > 0 and nr > 0 else (1.0 if ng == nr else 0.0)
    return max_rel, cos


def check_y(name: str, gpu_bits, ref_bits):
    max_rel, cos = y_metrics(gpu_bits, ref_bits)
    assert max_rel <= Y_MAX_REL, "%s: max rel %.4g > %g" % (name, max_rel, Y_MAX_REL)
    assert cos >= MIN_COS, "%s: cosine %.6f < %g" % (name, cos, MIN_COS)
    return max_rel, cos


@dataclass
class CaseReport:
    name: str
    layers_checked: List[int] = field(default_factory=list)
    xq_mismatch: int = 0
    xq_n: int = 0
    xq_near_boundary: int = 0
    hq_mismatch: int = 0
    hq_n: int = 0
    hq_t_max: float = 0.0
    y_max_rel: float = 0.0
    y_min_cos: float = 1.0
    z_cos: float = 1.0
    z_dist: float = 0.0
    z_dist_natural: float = 0.0
    natural: dict = field(default_factory=dict)
    z_max_rel: float = 0.0
    p10_cos_gpu: float = 1.0
    p10_cos_oracle: float = 1.0
    cal_max_rel: float = 0.0
    cal_tf_max_rel: float = 0.0
    saturated_codes: int = 0
    subnormal_codes: int = 0    # E4M3 codes with a zero exponent field and a nonzero mantissa
    zero_xq_rows: int = 0       # rows of XQ[0] that are all zero codes
    path: int = 0               # FRT_PATH_* bits of the plan
    seconds: float = 0.0


def run_case(cfg: FFNConfig, rows: Optional[Sequence[int]] = None, cal_rows: Optional[Sequence[int]] = None,
             check_layers: Optional[Sequence[int]] = None, nbatch: int = 4, flags: int = 0,
             gate_drift: bool = True, gate_hq: bool = True, edit_inputs=None) -> CaseReport:
    """Full parity procedure; rows / cal_rows select the evaluated / calibration
    rows (None = all); check_layers selects the teacher-forced layers (None = all);
    flags are plan flags; gate_drift gates the free-running chain and gate_hq the
    re-quantised HQ bytes (else both are reported only); edit_inputs(r0, y0)
    returns replaced evaluation inputs (bf16 bits), given to both sides."""
    t0 = time.time()
    rep = CaseReport(cfg.name)
    M, H, I, L, act = cfg.M, cfg.H, cfg.I, cfg.L, cfg.act
    rows_arg = rows
    rows = np.arange(M) if rows is None else np.asarray(sorted(rows))
    r0, y0 = datagen.eval_inputs(cfg)
    if edit_inputs is not None:
        r0, y0 = edit_inputs(r0, y0)
    cal = datagen.calib_batches(cfg, nbatch)
    if cal_rows is not None:
        cr = np.asarray(sorted(cal_rows))
        cal = [(r[cr], None if y is None else y[cr]) for r, y in cal]
    log("[case %s] M=%d H=%d I=%d L=%d act=%d rows=%d cal_rows=%d" % (
        cfg.name, M, H, I, L, act, len(rows), cal[0][0].shape[0]))

    plan = FFNPlan(M, H, I, L, act, cfg.eps, flags=flags)
    rep.path = plan.path()
    try:
        weight_scales = []
        norm_w = {}
        mods = {}
        norm_fuse = bool(flags & _abi.FRT_FLAG_NORM_FUSE)
        ada = bool(flags & _abi.FRT_FLAG_ADA_NORM)
        # quantised weights kept for the HQ mismatch analysis when they are
        # small; otherwise a layer is regenerated (seeded) if it has any
        keep_weights = 3 * I * H * L <= (1 << 31)
        kept_lw = {}

        def layer_lw(l):
            if l in kept_lw:
                return kept_lw[l]
            wg, wu, wd, wn = datagen.layer_weights(cfg, l)
            mod = datagen.modulation(cfg, l) if ada else None
            return oracle.LayerWeights.quantize(wg, wu, wd, wn, norm_fuse=norm_fuse, mod=mod)

        def provider(l):
            def get():
                wg, wu, wd, wn = datagen.layer_weights(cfg, l)
                plan.load_layer(l, wg, wu, wd, wn)
                mod = datagen.modulation(cfg, l) if ada else None
                if ada:
                    plan.set_modulation(l, *mod)
                lw = oracle.LayerWeights.quantize(wg, wu, wd, wn, norm_fuse=norm_fuse, mod=mod)
                names = ["up", "down"] if wg is None else ["gate", "up", "down"]
                refs = [lw.qu, lw.qd] if wg is None else [lw.qg, lw.qu, lw.qd]
                idx = [1, 2] if wg is None else [0, 1, 2]
                for nm, which, ref in zip(names, idx, refs):
                    got = plan.export_codes(l, which)
                    nbad = int(np.count_nonzero(got != ref))
                    assert nbad == 0, "layer %d %s weight codes: %d mismatches" % (l, nm, nbad)
                weight_scales.append((lw.s_g, lw.s_u, lw.s_d))
                norm_w[l] = lw.w_norm
                mods[l] = lw.mod
                if keep_weights:
                    kept_lw[l] = lw
                if L > 4 and (l % 4 == 3 or l == L - 1):
                    log("[case %s] layers 0..%d quantised and compared (%.1fs)" % (cfg.name, l, time.time() - t0))
                return lw
            return get

        # the valid fp32 orders' chains: from the stored record for the
        # large named workloads, else stepped here beside the oracle
        stored = stored_natural_drift(cfg, None if rows_arg is None else rows, cal_rows)
        nat = None if stored is not None else _natural.NaturalChains(r0[rows], None if y0 is None else y0[rows])

        # P-10: the same chain with unquantised fp32 activations (the
        # oracle's measurement-mode block) from the same input
        unq = {"r": r0[rows], "y": None if y0 is None else y0[rows]}

        def natural_step(li, lw, s_x, s_h):
            if nat is not None:
                nat.step(lw, act, cfg.eps, s_x, s_h)
            unq["r"], unq["y"], _, _ = oracle.block_measure(unq["r"], unq["y"], lw, act, cfg.eps)

        orc = oracle.calibrate_and_run((provider(l) for l in range(L)), act, cfg.eps,
                                       r0[rows], None if y0 is None else y0[rows], cal,
                                       keep_cal_states=True, post_layer=natural_step)
        log("[case %s] weights bit-exact; oracle chain done (%.1fs)" % (cfg.name, time.time() - t0))

        sc = plan.scales()
        for l in range(L):
            sg, su, sd = weight_scales[l]
            assert (sc[l, 1], sc[l, 2], sc[l, 4]) == (np.float32(sg), np.float32(su), np.float32(sd)), \
                "layer %d weight scales differ: gpu %s oracle %s" % (l, sc[l], weight_scales[l])

        # calibration on the GPU over the same batches, compared with the oracle
        plan.calibrate(cal)
        sc = plan.scales()
        rel_x = np.abs(sc[:, 0] / np.asarray(orc.s_x, np.float64) - 1)
        rel_h = np.abs(sc[:, 3] / np.asarray(orc.s_h, np.float64) - 1)
        rep.cal_max_rel = float(max(rel_x.max(), rel_h.max()))
        assert max(rel_x[0], rel_h[0]) <= CAL_RTOL_FIRST, "first-layer calibration scales differ by %.3g" % max(
            rel_x[0], rel_h[0])
        assert rep.cal_max_rel <= CAL_DRIFT_MAX, "calibration scales drift by %.3g" % rep.cal_max_rel
        # teacher-forced calibration: each checked layer measured from the
        # oracle's own measurement states entering it
        tf_layers = range(L) if check_layers is None else check_layers
        for l in tf_layers:
            plan.calibrate(orc.cal_states[l], layer_begin=l, layer_end=l + 1)
        sc = plan.scales()
        tf = [max(abs(sc[l, 0] / orc.s_x[l] - 1), abs(sc[l, 3] / orc.s_h[l] - 1)) for l in tf_layers]
        rep.cal_tf_max_rel = float(max(tf))
        assert rep.cal_tf_max_rel <= CAL_RTOL_FIRST, "per-layer calibration scales differ by %.3g" % rep.cal_tf_max_rel
        log("[case %s] calibration: chain drift %.2e, per-layer %.2e" % (cfg.name, rep.cal_max_rel, rep.cal_tf_max_rel))

        # the forward uses the oracle's scales (cache-hit path)
        plan.set_act_scales(orc.s_x, orc.s_h)
        plan.set_inputs(r0, y0)
        plan.capture()
        plan.replay()
        plan.sync()
        z_graph = to_np_u16(plan.z())
        yl_graph = to_np_u16(plan.y_slot(L))
        plan.replay()
        plan.sync()
        assert np.array_equal(to_np_u16(plan.z()), z_graph), "two graph replays differ"
        plan.forward()
        plan.sync()
        assert np.array_equal(to_np_u16(plan.z()), z_graph), "eager forward differs from graph replay"
        assert np.array_equal(to_np_u16(plan.y_slot(L)), yl_graph), "eager Y[L] differs from replay"
        # chain consistency of the free-running forward: every layer's R' and
        # XQ follow from the R and Y slots it started from (the oracle's
        # residual add and norm applied to the GPU's own slots), R' bit for
        # bit and XQ under the code rule, and Z from R[L] and Y[L].  This
        # holds on every path, including where a down GEMV forms the next
        # layer's R' and norm slice sums itself.
        ridx = torch.as_tensor(rows, device=plan.device)
        for l in range(L):
            r_in = to_np_u16(plan.r_slot(l)[ridx])
            y_in = to_np_u16(plan.y_slot(l)[ridx])
            inv_x = np.float32(np.float32(1.0) / np.float32(orc.s_x[l]))
            r_ref, x_pre, _ = oracle.add_rmsnorm_quant(r_in, y_in, norm_w[l], cfg.eps, 1.0, mod=mods[l])
            nb = int(np.count_nonzero(to_np_u16(plan.r_slot(l + 1)[ridx]) != r_ref))
            assert nb == 0, "free-running layer %d residual: %d bf16 mismatches against its own R and Y" % (l, nb)
            _, _, xq_ref = oracle.add_rmsnorm_quant(r_in, y_in, norm_w[l], cfg.eps, float(inv_x), mod=mods[l])
            xs = code_stats(to_np_u8(plan.xq_slot(l)[ridx]), xq_ref, (x_pre * inv_x).astype(np.float32))
            check_codes("free-running layer %d XQ" % l, xs, boundary_rule=True)
        z_own = oracle.final_hidden(to_np_u16(plan.r_slot(L)[ridx]), to_np_u16(plan.y_slot(L)[ridx]))
        nb = int(np.count_nonzero(z_graph[rows] != z_own))
        assert nb == 0, "Z: %d bf16 mismatches against the GPU's own R[L] + Y[L]" % nb
        # saturation invariant over every quantised slot
        for l in range(L):
            for t in (plan.xq_slot(l), plan.hq_slot(l)):
                codes = to_np_u8(t)
                assert not np.any((codes & 0x7F) == 0x7F), "NaN code in layer %d" % l
                rep.saturated_codes += int(np.count_nonzero((codes & 0x7F) == 0x7E))
                rep.subnormal_codes += int(np.count_nonzero(((codes & 0x78) == 0) & ((codes & 0x07) != 0)))
        xq0 = to_np_u8(plan.xq_slot(0)).reshape(M, H)
        rep.zero_xq_rows = int(np.count_nonzero(~np.any(xq0 & 0x7F, axis=1)))
        z_ref = oracle.final_hidden(orc.r[L], orc.y[L])
        rep.z_max_rel, rep.z_cos = y_metrics(z_graph[rows], z_ref)
        rep.z_dist = _natural.cos_distance(z_graph[rows], z_ref)
        rep.natural = stored if stored is not None else nat.distances(z_ref)
        rep.z_dist_natural = max(rep.natural.values())
        z_unq = oracle.final_hidden(unq["r"], unq["y"])
        _, rep.p10_cos_gpu = y_metrics(z_graph[rows], z_unq)
        _, rep.p10_cos_oracle = y_metrics(z_ref, z_unq)
        log("[case %s] P-10 (FP8 chain vs unquantised activations): Z cosine GPU %.6f, oracle %.6f" % (
            cfg.name, rep.p10_cos_gpu, rep.p10_cos_oracle))
        log("[case %s] graph == eager; Z cos %.6f max rel %.3g; drift %.3g, valid fp32 orders %s%s" % (
            cfg.name, rep.z_cos, rep.z_max_rel, rep.z_dist,
            " ".join("%s %.3g" % kv for kv in sorted(rep.natural.items())), " (stored)" if stored else ""))
        if gate_drift:
            assert rep.z_cos >= MIN_COS or rep.z_dist <= DRIFT_FACTOR * rep.z_dist_natural + DRIFT_FLOOR, \
                "free-running Z cosine %.6f < %g and drift %.3g > %g x the valid orders' largest %.3g" % (
                    rep.z_cos, MIN_COS, rep.z_dist, DRIFT_FACTOR, rep.z_dist_natural)

        # teacher-forced per-block checks
        idx = torch.as_tensor(rows, device=plan.device)
        layers = range(L) if check_layers is None else check_layers
        for l in layers:
            with torch.cuda.stream(plan.stream):
                plan.r_slot(l).index_copy_(0, idx, torch.from_numpy(orc.r[l].view(np.int16)).to(plan.device))
                if orc.y[l] is None:
                    plan.y_slot(l).index_fill_(0, idx, 0)
                else:
                    plan.y_slot(l).index_copy_(0, idx, torch.from_numpy(orc.y[l].view(np.int16)).to(plan.device))
            plan.sync()
            plan.forward_range(l, l + 1)
            plan.sync()
            r_g = to_np_u16(plan.r_slot(l + 1)[idx])
            xq_g = to_np_u8(plan.xq_slot(l)[idx])
            hq_g = to_np_u8(plan.hq_slot(l)[idx])
            y_g = to_np_u16(plan.y_slot(l + 1)[idx])
            nb = int(np.count_nonzero(r_g != orc.r[l + 1]))
            assert nb == 0, "layer %d residual: %d bf16 mismatches" % (l, nb)
            # oracle pre-rounding value of XQ for the boundary report
            _, x_pre, _ = oracle.add_rmsnorm_quant(orc.r[l], orc.y[l], norm_w[l], cfg.eps, 1.0, mod=mods[l])
            inv_x = np.float32(np.float32(1.0) / np.float32(orc.s_x[l]))
            xs = code_stats(xq_g, orc.xq[l], (x_pre * inv_x).astype(np.float32))
            check_codes("layer %d XQ" % l, xs, boundary_rule=True)
            hs = code_stats(hq_g, orc.hq[l])
            if hs.mismatches:
                nh, tmax = _hq_explain.explain(orc.xq[l], hq_g, orc.hq[l], layer_lw(l), act,
                                               orc.s_x[l], orc.s_h[l])
                rep.hq_t_max = max(rep.hq_t_max, tmax)
                log("[case %s] layer %d HQ: %d mismatches, largest accumulation error needed %.3g units"
                    % (cfg.name, l, nh, tmax))
            if gate_hq:
                check_codes("layer %d HQ" % l, hs)
                if hs.mismatches and rep.hq_t_max > _hq_explain.T_MAX_EXPLAINED:
                    raise CodeToleranceMiss(
                        "layer %d HQ: a mismatch needs an accumulation error of %.3g units (> %g): "
                        "not explained by fp32 accumulation" % (l, rep.hq_t_max, _hq_explain.T_MAX_EXPLAINED))
            mr, cs = check_y("layer %d Y" % l, y_g, orc.y[l + 1])
            rep.layers_checked.append(l)
            rep.xq_mismatch += xs.mismatches
            rep.xq_n += xs.n
            rep.xq_near_boundary += max(0, xs.near_boundary)
            rep.hq_mismatch += hs.mismatches
            rep.hq_n += hs.n
            rep.y_max_rel = max(rep.y_max_rel, mr)
            rep.y_min_cos = min(rep.y_min_cos, cs)
        log("[case %s] per-block: XQ %d/%d (near boundary %d), HQ %d/%d (largest error needed %.3g units), "
            "Y max rel %.3g min cos %.6f"
            % (cfg.name, rep.xq_mismatch, rep.xq_n, rep.xq_near_boundary, rep.hq_mismatch, rep.hq_n,
               rep.hq_t_max, rep.y_max_rel, rep.y_min_cos))
    finally:
        plan.close()
    rep.seconds = time.time() - t0
    return rep


def run_permutation(cfg: FFNConfig, flags: int = 0, seed: int = 7, layers: Optional[int] = None) -> int:
    """Row independence on the GPU (one plan, one kernel path): the chain run
    on the evaluation input with its rows permuted must give every slot
    (R, XQ, HQ, Y per layer, and Z) permuted the same way, bit for bit.
    Scales come from the GPU's own calibration pass (any fixed scales do).
    Returns the number of layers compared."""
    M, H, I = cfg.M, cfg.H, cfg.I
    L = cfg.L if layers is None else min(cfg.L, layers)
    r0, y0 = datagen.eval_inputs(cfg)
    perm = np.random.default_rng(seed).permutation(M)
    log("[perm %s] M=%d H=%d I=%d L=%d flags=%d" % (cfg.name, M, H, I, L, flags))
    plan = FFNPlan(M, H, I, L, cfg.act, cfg.eps, flags=flags)
    try:
        for l in range(L):
            plan.load_layer(l, *datagen.layer_weights(cfg, l))
        plan.calibrate(datagen.calib_batches(cfg, 1))

        def run(r, y):
            plan.set_inputs(r, y)
            plan.forward()
            plan.sync()
            out = []
            for l in range(L):
                out.append((to_np_u16(plan.r_slot(l + 1)), to_np_u8(plan.xq_slot(l)), to_np_u8(plan.hq_slot(l)),
                            to_np_u16(plan.y_slot(l + 1))))
            return out, to_np_u16(plan.z())

        base, z = run(r0, y0)
        prm, zp = run(np.ascontiguousarray(r0[perm]), None if y0 is None else np.ascontiguousarray(y0[perm]))
        for l in range(L):
            for name, a, b in zip(("R", "XQ", "HQ", "Y"), base[l], prm[l]):
                nb = int(np.count_nonzero(a[perm] != b))
                assert nb == 0, "layer %d %s: %d elements differ after the row permutation" % (l, name, nb)
        assert np.array_equal(z[perm], zp), "Z differs after the row permutation"
    finally:
        plan.close()
    log("[perm %s] %d layers: every slot permuted bit for bit" % (cfg.name, L))
    return L
