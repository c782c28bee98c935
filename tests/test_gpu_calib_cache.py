"""Calibration cache on the GPU: a miss measures on one plan and writes the
JSON file; a second plan over the same weights hits it, installs the same
scale bits and produces the same output bits."""
import os

import numpy as np
import pytest

from realtime_transformer_amd import calib_cache, datagen
from realtime_transformer_amd.configs import FFNConfig, ACT_GEGLU_TANH
from realtime_transformer_amd.plan import FFNPlan, to_np_u16

pytestmark = pytest.mark.gpu


def _plan_with_weights(cfg):
    plan = FFNPlan(cfg.M, cfg.H, cfg.I, cfg.L, cfg.act, cfg.eps)
    hasher = calib_cache.CkptHasher(cfg.H, cfg.I, cfg.L, cfg.act, cfg.eps)
    for l in range(cfg.L):
        w = datagen.layer_weights(cfg, l)
        plan.load_layer(l, *w)
        hasher.add_layer(w)
    return plan, hasher.hexdigest()


def _forward_z(plan, r0, y0):
    plan.set_inputs(r0, y0)
    plan.forward()
    plan.sync()
    return to_np_u16(plan.z())


def test_cache_miss_then_hit(tmp_path):
    cfg = FFNConfig(112, "small_cache_112", 33, 256, 512, 3, ACT_GEGLU_TANH)
    r0, y0 = datagen.eval_inputs(cfg)
    cal = datagen.calib_batches(cfg, 2)
    a, h = _plan_with_weights(cfg)
    try:
        assert calib_cache.calibrate_cached(a, h, cal, root=str(tmp_path)) is False
        assert os.path.exists(calib_cache.cache_path(h, cfg.M, str(tmp_path)))
        sa = a.scales()
        za = _forward_z(a, r0, y0)
    finally:
        a.close()
    b, h2 = _plan_with_weights(cfg)
    try:
        assert h2 == h
        assert calib_cache.calibrate_cached(b, h, None, root=str(tmp_path)) is True
        sb = b.scales()
        assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
        zb = _forward_z(b, r0, y0)
        assert np.array_equal(za, zb)
    finally:
        b.close()
