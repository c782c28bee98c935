"""The forward with its scratch in the library's static device array
(frt_ffn_forward_range_static_scratch, for callers that cannot allocate)
against the workspace-scratch forward (frt_ffn_forward_range), through the
C ABI: every slot bit for bit, on two calls in a row, the second on a smaller
plan (the array then holds the first call's contents)."""
import numpy as np
import pytest

from realtime_transformer_amd import _abi, datagen
from realtime_transformer_amd.configs import FFNConfig, ACT_GEGLU_TANH, ACT_SWIGLU, ACT_GELU_TANH
from realtime_transformer_amd.plan import FFNPlan, to_np_u16, to_np_u8

pytestmark = pytest.mark.gpu


def _slots(plan, L, mx):
    out = [to_np_u16(plan.z())]
    for l in range(L):
        xq = plan.xq_mx(l) if mx else (plan.xq_slot(l),)
        hq = plan.hq_mx(l) if mx else (plan.hq_slot(l),)
        out += [to_np_u16(plan.r_slot(l + 1))] + [to_np_u8(t) for t in xq + hq] + [to_np_u16(plan.y_slot(l + 1))]
    return out


def _clobber(plan, L):
    # every byte of each XQ and HQ slot (MXFP4: codes, exponents and padding)
    for l in range(L):
        plan._view(plan.io.xq_slots + l * plan.io.stride_xq, plan.io.stride_xq).fill_(0x7F)
        plan._view(plan.io.hq_slots + l * plan.io.stride_hq, plan.io.stride_hq).fill_(0x7F)


def _compare(cfg, flags=0):
    print("[no-alloc] %s M=%d H=%d I=%d L=%d flags=%d" % (cfg.name, cfg.M, cfg.H, cfg.I, cfg.L, flags), flush=True)
    plan = FFNPlan(cfg.M, cfg.H, cfg.I, cfg.L, cfg.act, cfg.eps, flags=flags)
    try:
        for l in range(cfg.L):
            plan.load_layer(l, *datagen.layer_weights(cfg, l))
        if not flags & _abi.FRT_FLAG_MXFP4:  # MXFP4 takes its block scales from the data
            plan.calibrate(datagen.calib_batches(cfg, 1))
        r0, y0 = datagen.eval_inputs(cfg)
        plan.set_inputs(r0, y0)
        _abi.frt_ffn_forward_range(plan.plan, 0, cfg.L, plan.s)
        plan.sync()
        mx = bool(flags & _abi.FRT_FLAG_MXFP4)
        ref = _slots(plan, cfg.L, mx)
        # clobber the outputs, then the static-scratch variant from the same inputs
        _clobber(plan, cfg.L)
        plan.set_inputs(r0, y0)
        _abi.frt_ffn_forward_range_static_scratch(plan.plan, 0, cfg.L, plan.s)
        plan.sync()
        got = _slots(plan, cfg.L, mx)
        for i, (a, b) in enumerate(zip(ref, got)):
            assert np.array_equal(a, b), "slot %d differs between the two forwards" % i
    finally:
        plan.close()


def test_static_scratch_forward_matches_workspace_forward_two_calls():
    # first a prefill-shaped plan whose down GEMM splits K (partials in the
    # array), then a smaller decode-shaped plan (the whole-column down GEMV's
    # slice sums), so the second call finds the first call's bytes in the
    # array; then an MXFP4 decode plan on the same path
    _compare(FFNConfig(121, "noalloc_prefill", 300, 512, 2048, 2, ACT_GEGLU_TANH))
    _compare(FFNConfig(122, "noalloc_decode", 1, 1024, 4096, 3, ACT_SWIGLU))
    _compare(FFNConfig(165, "noalloc_decode_mx", 2, 512, 2048, 2, ACT_GEGLU_TANH), flags=_abi.FRT_FLAG_MXFP4)


def test_static_scratch_rejects_plans_beyond_its_size(monkeypatch):
    # M=64, H=8192 with the down GEMV split 16 ways: 32 MiB of fp32 partials
    monkeypatch.setenv("FRT_GEMV_DOWN_SPLIT", "16")
    cfg = FFNConfig(123, "noalloc_big", 64, 8192, 2048, 1, ACT_GELU_TANH)
    print("[no-alloc] rejection M=%d H=%d I=%d split 16" % (cfg.M, cfg.H, cfg.I), flush=True)
    plan = FFNPlan(cfg.M, cfg.H, cfg.I, cfg.L, cfg.act, cfg.eps)
    try:
        for l in range(cfg.L):
            plan.load_layer(l, *datagen.layer_weights(cfg, l))
        plan.set_act_scales([0.01] * cfg.L, [0.01] * cfg.L)
        with pytest.raises(_abi.FrtError) as e:
            _abi.frt_ffn_forward_range_static_scratch(plan.plan, 0, cfg.L, plan.s)
        if e.value.status != _abi.FRT_ERR_UNSUPPORTED or "static array" not in _abi.frt_last_error():
            raise AssertionError("unexpected error: %s" % _abi.frt_last_error())
    finally:
        plan.close()
