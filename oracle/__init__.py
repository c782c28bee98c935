"""Python marshalling for the plain CPU oracle in ``oracle.c``.

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``.  The product package
(``realtime_transformer_amd``) never imports this module, and this module never
imports the product package; the only code both sides share is the seeded input
generator (``realtime_transformer_amd.datagen``), which holds none of the
method's arithmetic.

All arithmetic lives in ``oracle.c``.  This file only moves numpy arrays in and
out and strings the per-layer steps together in the pages' order:
quantise weights at load, calibrate (measurement pass, then static scales),
then run the block layer after layer (FlashRT architecture doc, "predict()
flow": weights -> calibration -> capture -> replay).

Array conventions: bf16 tensors are ``numpy.uint16`` holding the bf16 bit
pattern; E4M3 tensors are ``numpy.uint8`` codes; weights use the nn.Linear
layout ``[out, in]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Callable, Iterable, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ACT_GEGLU_TANH = 0
ACT_SWIGLU = 1
ACT_GELU_TANH = 2

_c_u8p = ctypes.POINTER(ctypes.c_uint8)
_c_u16p = ctypes.POINTER(ctypes.c_uint16)
_c_f32p = ctypes.POINTER(ctypes.c_float)
_c_f64p = ctypes.POINTER(ctypes.c_double)
_c_i32p = ctypes.POINTER(ctypes.c_int32)


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (ISO C11, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-pthread", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.orc_bf16_round.restype = ctypes.c_uint16
        L.orc_bf16_round.argtypes = [ctypes.c_float]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode_array.argtypes = [_c_f32p, _c_u8p, ctypes.c_int64]
        L.orc_e4m3_decode_array.argtypes = [_c_u8p, _c_f64p, ctypes.c_int64]
        L.orc_bf16_round_array.argtypes = [_c_f32p, _c_u16p, ctypes.c_int64]
        L.orc_gelu_tanh.restype = ctypes.c_double
        L.orc_gelu_tanh.argtypes = [ctypes.c_double]
        L.orc_silu.restype = ctypes.c_double
        L.orc_silu.argtypes = [ctypes.c_double]
        L.orc_act_f32.restype = ctypes.c_float
        L.orc_act_f32.argtypes = [ctypes.c_int, ctypes.c_float]
        L.orc_gemm_e4m3.restype = ctypes.c_int
        L.orc_gemm_e4m3.argtypes = [ctypes.c_int] * 3 + [_c_u8p, _c_u8p, _c_f32p, ctypes.c_int]
        L.orc_scale_from_amax.restype = ctypes.c_float
        L.orc_scale_from_amax.argtypes = [ctypes.c_float]
        L.orc_quant_tensor.restype = ctypes.c_float
        L.orc_quant_tensor.argtypes = [_c_u16p, ctypes.c_int64, _c_u8p]
        L.orc_quant_tensor_mt.restype = ctypes.c_float
        L.orc_quant_tensor_mt.argtypes = [_c_u16p, ctypes.c_int64, _c_u8p, ctypes.c_int]
        L.orc_quant_tensor_fold.restype = ctypes.c_float
        L.orc_quant_tensor_fold.argtypes = [_c_u16p, ctypes.c_int64, ctypes.c_int64, _c_u16p, _c_u8p,
                                            ctypes.c_int]
        L.orc_add_rmsnorm_quant.restype = None
        L.orc_add_rmsnorm_quant.argtypes = [ctypes.c_int, ctypes.c_int, _c_u16p, _c_u16p, _c_u16p,
                                            _c_u16p, _c_u16p, ctypes.c_float, ctypes.c_float, _c_u16p,
                                            _c_f32p, _c_u8p, ctypes.c_int]
        L.orc_gateup.restype = ctypes.c_int
        L.orc_gateup.argtypes = [ctypes.c_int] * 4 + [_c_u8p, _c_u8p, _c_u8p, ctypes.c_float,
                                                      ctypes.c_float, ctypes.c_float, _c_f32p,
                                                      _c_u8p, ctypes.c_int]
        L.orc_gateup_epilogue.restype = None
        L.orc_gateup_epilogue.argtypes = [ctypes.c_int64, ctypes.c_int, _c_f32p, _c_f32p, ctypes.c_float,
                                          ctypes.c_float, ctypes.c_float, _c_f32p, _c_u8p]
        L.orc_down_epilogue.restype = None
        L.orc_down_epilogue.argtypes = [ctypes.c_int64, _c_f32p, ctypes.c_float, _c_u16p]
        L.orc_down.restype = ctypes.c_int
        L.orc_down.argtypes = [ctypes.c_int] * 3 + [_c_u8p, _c_u8p, ctypes.c_float, _c_u16p,
                                                    ctypes.c_int]
        L.orc_block.restype = ctypes.c_int
        L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_decode.restype = ctypes.c_double
        L.orc_e2m1_encode.argtypes = [ctypes.c_double]
        L.orc_e2m1_encode.restype = ctypes.c_uint8
        L.orc_mx_scale_exp.argtypes = [ctypes.c_double]
        L.orc_mx_scale_exp.restype = ctypes.c_int
        L.orc_mxfp4_quant_rows.argtypes = [_c_f32p, ctypes.c_int64, ctypes.c_int64, _c_u8p, _c_u8p]
        L.orc_mxfp4_quant_rows.restype = None
        L.orc_mxfp4_quant_weight.argtypes = [_c_u16p, ctypes.c_int64, ctypes.c_int64, _c_u16p, _c_u8p, _c_u8p,
                                             ctypes.c_int]
        L.orc_mxfp4_quant_weight.restype = ctypes.c_int
        L.orc_mxfp4_gemm.argtypes = [ctypes.c_int] * 3 + [_c_u8p] * 4 + [_c_f32p, ctypes.c_int]
        L.orc_mxfp4_gemm.restype = ctypes.c_int
        L.orc_block_mxfp4.argtypes = ([ctypes.c_int] * 4 + [ctypes.c_float] + [_c_u16p] * 5 + [_c_f32p] +
                                      [_c_u8p] * 6 + [_c_u16p] + [_c_u8p] * 4 + [_c_u16p, ctypes.c_int])
        L.orc_block_mxfp4.restype = ctypes.c_int
        L.orc_rope_table.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, _c_f32p]
        L.orc_rope_table.restype = None
        L.orc_qkv_epilogue.argtypes = ([ctypes.c_int] * 4 + [_c_f32p, ctypes.c_float, _c_i32p, _c_f32p,
                                        ctypes.c_int, _c_u16p, _c_u16p, _c_u16p])
        L.orc_qkv_epilogue.restype = ctypes.c_int
        L.orc_block.argtypes = ([ctypes.c_int] * 4 + [ctypes.c_float, _c_u16p, _c_u16p, _c_u16p, _c_u16p,
                                                     _c_u16p, _c_u8p, _c_u8p, _c_u8p] + [ctypes.c_float] * 5
                                + [_c_u16p, _c_u8p, _c_u8p, _c_u16p, ctypes.c_int])
        L.orc_block_measure.restype = ctypes.c_int
        L.orc_block_measure.argtypes = ([ctypes.c_int] * 4 + [ctypes.c_float, _c_u16p, _c_u16p,
                                                             _c_u16p, _c_u16p, _c_u16p, _c_u8p, _c_u8p,
                                                             _c_u8p]
                                        + [ctypes.c_float] * 3
                                        + [_c_u16p, _c_u16p, _c_f32p, _c_f32p, ctypes.c_int])
        _lib = L
    return _lib


def default_threads() -> int:
    """Host threads the oracle uses: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _p(a: Optional[np.ndarray], ptype):
    if a is None:
        return ctypes.cast(None, ptype)
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ptype)


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _u8(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint8, a.dtype
    return a


# --------------------------------------------------------------------------
# scalar codecs (bulk forms for tests)
# --------------------------------------------------------------------------

def e4m3_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_e4m3_encode_array(_p(x, _c_f32p), _p(out, _c_u8p), x.size)
    return out


def e4m3_decode(c) -> np.ndarray:
    c = _u8(np.asarray(c, dtype=np.uint8))
    out = np.empty(c.shape, dtype=np.float64)
    lib().orc_e4m3_decode_array(_p(c, _c_u8p), _p(out, _c_f64p), c.size)
    return out


def bf16_round(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_bf16_round_array(_p(x, _c_f32p), _p(out, _c_u16p), x.size)
    return out


def bf16_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact: the bits become the top half)."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    assert np.little_endian
    out = np.zeros(b.shape + (2,), dtype=np.uint16)
    out[..., 1] = b  # little-endian: the second half-word is the high half
    return out.view(np.float32).reshape(b.shape)


def gelu_tanh(z: float) -> float:
    return lib().orc_gelu_tanh(float(z))


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


def act_f32(kind_is_silu: bool, z: float) -> float:
    return lib().orc_act_f32(1 if kind_is_silu else 0, float(z))


def scale_from_amax(amax: float) -> float:
    return lib().orc_scale_from_amax(float(amax))


# --------------------------------------------------------------------------
# GEMM, weight quantisation, block steps
# --------------------------------------------------------------------------

def gemm_e4m3(a_codes, b_codes, nthreads: Optional[int] = None) -> np.ndarray:
    """f32(exact sum_k dec(a[m,k]) * dec(b[n,k])) for a [M,K], b [N,K]."""
    a = _u8(a_codes)
    b = _u8(b_codes)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    out = np.empty((M, N), dtype=np.float32)
    rc = lib().orc_gemm_e4m3(M, N, K, _p(a, _c_u8p), _p(b, _c_u8p), _p(out, _c_f32p),
                             nthreads or default_threads())
    if rc != 0:
        raise ValueError("K too large for the exact int64 sum")
    return out


def quant_tensor(w_bf16, nthreads: Optional[int] = None) -> tuple:
    """Per-tensor E4M3 quantisation of a bf16 tensor -> (codes, scale)."""
    w = _u16(w_bf16)
    codes = np.empty(w.shape, dtype=np.uint8)
    s = lib().orc_quant_tensor_mt(_p(w, _c_u16p), w.size, _p(codes, _c_u8p),
                                  nthreads or default_threads())
    return codes, float(np.float32(s))


def quant_tensor_fold(w_bf16, colw_bf16, nthreads: Optional[int] = None) -> tuple:
    """Per-tensor E4M3 quantisation of f32(w[i][k] * colw[k]) for a bf16
    [rows][cols] tensor and a bf16 [cols] column factor (norm fusion) ->
    (codes, scale)."""
    w = _u16(w_bf16)
    c = _u16(colw_bf16)
    rows, cols = w.shape
    assert c.shape == (cols,)
    codes = np.empty(w.shape, dtype=np.uint8)
    s = lib().orc_quant_tensor_fold(_p(w, _c_u16p), rows, cols, _p(c, _c_u16p), _p(codes, _c_u8p),
                                    nthreads or default_threads())
    return codes, float(np.float32(s))


def add_rmsnorm_quant(r_prev, y_prev, w_norm, eps: float, inv_x: float,
                      nthreads: Optional[int] = None, mod=None):
    """-> (r_out bf16 [M,H], x fp32 [M,H], xq codes [M,H]).  ``mod`` =
    (scale, shift) bf16 [H] selects AdaRMSNorm modulation instead of w_norm."""
    r = _u16(r_prev)
    M, H = r.shape
    y = None if y_prev is None else _u16(y_prev)
    w = _u16(w_norm)
    ms, mh = (None, None) if mod is None else (_u16(mod[0]), _u16(mod[1]))
    r_out = np.empty((M, H), np.uint16)
    x = np.empty((M, H), np.float32)
    xq = np.empty((M, H), np.uint8)
    lib().orc_add_rmsnorm_quant(M, H, _p(r, _c_u16p), _p(y, _c_u16p), _p(w, _c_u16p), _p(ms, _c_u16p),
                                _p(mh, _c_u16p), float(eps), float(inv_x), _p(r_out, _c_u16p),
                                _p(x, _c_f32p), _p(xq, _c_u8p), nthreads or default_threads())
    return r_out, x, xq


def gateup(xq, qg, qu, act: int, alpha_g: float, alpha_u: float, inv_h: float,
           nthreads: Optional[int] = None):
    """-> (h fp32 [M,I], hq codes [M,I])."""
    xq = _u8(xq)
    qu = _u8(qu)
    M, H = xq.shape
    I = qu.shape[0]
    qg = None if act == ACT_GELU_TANH else _u8(qg)
    h = np.empty((M, I), np.float32)
    hq = np.empty((M, I), np.uint8)
    rc = lib().orc_gateup(M, H, I, act, _p(xq, _c_u8p), _p(qg, _c_u8p), _p(qu, _c_u8p),
                          float(alpha_g), float(alpha_u), float(inv_h), _p(h, _c_f32p),
                          _p(hq, _c_u8p), nthreads or default_threads())
    if rc:
        raise RuntimeError("orc_gateup failed (%d)" % rc)
    return h, hq


def gateup_epilogue(Ag, Au, act: int, alpha_g: float, alpha_u: float, inv_h: float):
    """Step-2 epilogue on given fp32 accumulators -> (h fp32, hq codes)."""
    Au = np.ascontiguousarray(Au, dtype=np.float32)
    Ag = None if act == ACT_GELU_TANH else np.ascontiguousarray(Ag, dtype=np.float32)
    h = np.empty(Au.shape, np.float32)
    hq = np.empty(Au.shape, np.uint8)
    lib().orc_gateup_epilogue(Au.size, act, _p(Ag, _c_f32p), _p(Au, _c_f32p), float(alpha_g),
                              float(alpha_u), float(inv_h), _p(h, _c_f32p), _p(hq, _c_u8p))
    return h, hq


def down_epilogue(Ad, alpha_d: float) -> np.ndarray:
    """Step-3 epilogue on given fp32 accumulators -> bf16 bits."""
    Ad = np.ascontiguousarray(Ad, dtype=np.float32)
    y = np.empty(Ad.shape, np.uint16)
    lib().orc_down_epilogue(Ad.size, _p(Ad, _c_f32p), float(alpha_d), _p(y, _c_u16p))
    return y


def down(hq, qd, alpha_d: float, nthreads: Optional[int] = None) -> np.ndarray:
    hq = _u8(hq)
    qd = _u8(qd)
    M, I = hq.shape
    H = qd.shape[0]
    y = np.empty((M, H), np.uint16)
    rc = lib().orc_down(M, H, I, _p(hq, _c_u8p), _p(qd, _c_u8p), float(alpha_d),
                        _p(y, _c_u16p), nthreads or default_threads())
    if rc:
        raise RuntimeError("orc_down failed (%d)" % rc)
    return y


ONES_BF16 = 0x3F80  # bf16 1.0


@dataclass
class LayerWeights:
    """One layer's quantised weights as the oracle holds them.  ``mod`` =
    (scale, shift) bf16 [H] selects AdaRMSNorm modulation for the norm step
    (then w_norm is unused)."""
    qg: Optional[np.ndarray]  # [I,H] codes (None when non-gated)
    qu: np.ndarray            # [I,H] codes
    qd: np.ndarray            # [H,I] codes
    w_norm: np.ndarray        # [H] bf16 bits
    s_g: float
    s_u: float
    s_d: float
    mod: Optional[tuple] = None

    @staticmethod
    def quantize(w_gate, w_up, w_down, w_norm, norm_fuse: bool = False, mod=None) -> "LayerWeights":
        """norm_fuse: fold w_norm into the gate/up matrices (per input
        column) before quantising and normalise with a unit weight."""
        w_norm = _u16(w_norm)
        if norm_fuse:
            qg, s_g = (None, 1.0) if w_gate is None else quant_tensor_fold(w_gate, w_norm)
            qu, s_u = quant_tensor_fold(w_up, w_norm)
            w_norm = np.full(w_norm.shape, ONES_BF16, np.uint16)
        else:
            qg, s_g = (None, 1.0) if w_gate is None else quant_tensor(w_gate)
            qu, s_u = quant_tensor(w_up)
        qd, s_d = quant_tensor(w_down)
        mod = None if mod is None else (_u16(mod[0]), _u16(mod[1]))
        return LayerWeights(qg, qu, qd, w_norm, s_g, s_u, s_d, mod)

    def mod_ptrs(self):
        return (None, None) if self.mod is None else self.mod


def block(r_prev, y_prev, lw: LayerWeights, act: int, eps: float, s_x: float, s_h: float,
          nthreads: Optional[int] = None):
    """One FFN block -> (r_out, xq, hq, y_out)."""
    r = _u16(r_prev)
    M, H = r.shape
    I = lw.qu.shape[0]
    y = None if y_prev is None else _u16(y_prev)
    r_out = np.empty((M, H), np.uint16)
    xq = np.empty((M, H), np.uint8)
    hq = np.empty((M, I), np.uint8)
    y_out = np.empty((M, H), np.uint16)
    ms, mh = lw.mod_ptrs()
    rc = lib().orc_block(M, H, I, act, float(eps), _p(r, _c_u16p), _p(y, _c_u16p),
                         _p(lw.w_norm, _c_u16p), _p(ms, _c_u16p), _p(mh, _c_u16p), _p(lw.qg, _c_u8p),
                         _p(lw.qu, _c_u8p),
                         _p(lw.qd, _c_u8p), lw.s_g, lw.s_u, lw.s_d, float(s_x), float(s_h),
                         _p(r_out, _c_u16p), _p(xq, _c_u8p), _p(hq, _c_u8p), _p(y_out, _c_u16p),
                         nthreads or default_threads())
    if rc:
        raise RuntimeError("orc_block failed (%d)" % rc)
    return r_out, xq, hq, y_out


def block_measure(r_prev, y_prev, lw: LayerWeights, act: int, eps: float,
                  nthreads: Optional[int] = None):
    """Calibration measurement pass of one block -> (r_out, y_out, amax_x, amax_h)."""
    r = _u16(r_prev)
    M, H = r.shape
    I = lw.qu.shape[0]
    y = None if y_prev is None else _u16(y_prev)
    r_out = np.empty((M, H), np.uint16)
    y_out = np.empty((M, H), np.uint16)
    ax = ctypes.c_float(0.0)
    ah = ctypes.c_float(0.0)
    ms, mh = lw.mod_ptrs()
    rc = lib().orc_block_measure(M, H, I, act, float(eps), _p(r, _c_u16p), _p(y, _c_u16p),
                                 _p(lw.w_norm, _c_u16p), _p(ms, _c_u16p), _p(mh, _c_u16p),
                                 _p(lw.qg, _c_u8p), _p(lw.qu, _c_u8p),
                                 _p(lw.qd, _c_u8p), lw.s_g, lw.s_u, lw.s_d, _p(r_out, _c_u16p),
                                 _p(y_out, _c_u16p), ctypes.byref(ax), ctypes.byref(ah),
                                 nthreads or default_threads())
    if rc:
        raise RuntimeError("orc_block_measure failed (%d)" % rc)
    return r_out, y_out, float(ax.value), float(ah.value)


def final_hidden(r_last, y_last) -> np.ndarray:
    """Z = bf16(f32(R[L] + Y[L])) (the residual add after the last block)."""
    s = bf16_to_f32(r_last) + bf16_to_f32(y_last)
    return bf16_round(s)


@dataclass
class ChainResult:
    s_x: List[float]
    s_h: List[float]
    amax_x: List[float]
    amax_h: List[float]
    r: List[np.ndarray]   # R[0..L]
    y: List[np.ndarray]   # Y[0..L]
    xq: List[np.ndarray]  # XQ[0..L-1]
    hq: List[np.ndarray]  # HQ[0..L-1]
    weights: List[Optional[LayerWeights]]
    cal_states: List[list] = None  # per layer: the (r, y) batches entering it (measure mode)


def calibrate_and_run(layers: Iterable[Callable[[], LayerWeights]], act: int, eps: float,
                      r0, y0, calib_batches: Sequence[tuple], keep_weights: bool = False,
                      act_scales: Optional[Sequence[tuple]] = None,
                      nthreads: Optional[int] = None, keep_cal_states: bool = False,
                      post_layer: Optional[Callable] = None) -> ChainResult:
    """Layer-major chain: for each layer, measure the calibration batches
    (amax of the gate/up input and of the down input over all batches, rows
    and elements), derive the static scales s = f32(amax/448), then run the
    quantised block on the evaluation state.  ``layers`` yields one callable
    per layer that returns its quantised weights, so huge chains can stream
    their weights.  ``act_scales`` (per layer (s_x, s_h)) skips the
    measurement and uses the given scales (the calibration cache-hit path).
    ``post_layer(li, lw, s_x, s_h)`` is called after each layer.
    """
    cal_states = [(_u16(r), None if y is None else _u16(y)) for r, y in calib_batches]
    res = ChainResult([], [], [], [], [_u16(r0)], [None if y0 is None else _u16(y0)], [], [], [], [])
    for li, get_w in enumerate(layers):
        lw = get_w()
        if keep_cal_states:
            res.cal_states.append(list(cal_states))
        if act_scales is None:
            ax = 0.0
            ah = 0.0
            nxt = []
            for (r, y) in cal_states:
                r2, y2, bx, bh = block_measure(r, y, lw, act, eps, nthreads)
                ax = max(ax, bx)
                ah = max(ah, bh)
                nxt.append((r2, y2))
            cal_states = nxt
            s_x = scale_from_amax(ax)
            s_h = scale_from_amax(ah)
        else:
            ax = ah = float("nan")
            s_x, s_h = act_scales[li]
        r_out, xq, hq, y_out = block(res.r[-1], res.y[-1], lw, act, eps, s_x, s_h, nthreads)
        res.s_x.append(s_x)
        res.s_h.append(s_h)
        res.amax_x.append(ax)
        res.amax_h.append(ah)
        res.r.append(r_out)
        res.y.append(y_out)
        res.xq.append(xq)
        res.hq.append(hq)
        res.weights.append(lw if keep_weights else None)
        if post_layer is not None:
            post_layer(li, lw, s_x, s_h)
    return res


# ---------------------------------------------------------------------------
# Attention input: fused QKV projection + split + rotary embedding
# (FlashRT architecture doc, "Kernel library": the "qkv split + RoPE" fusion;
# itsolotime article section 5.2: the FusedQKV weight of the Pi0/Pi0.5 specs)
# ---------------------------------------------------------------------------

def rope_table(P: int, hd: int, base: float) -> np.ndarray:
    """[P, hd/2, 2] float32 (cos, sin) of p * base^(-2i/hd), fp64 then rounded."""
    assert hd % 2 == 0 and P >= 1
    out = np.empty((P, hd // 2, 2), np.float32)
    lib().orc_rope_table(int(P), int(hd), float(base), _p(out, _c_f32p))
    return out


def qkv_epilogue(A, alpha: float, nq: int, nkv: int, hd: int, pos, table):
    """fp32 GEMM result [M, (nq+2nkv)*hd] -> bf16 (Q [M,nq,hd], K [M,nkv,hd], V [M,nkv,hd])."""
    A = np.ascontiguousarray(A, np.float32)
    M = A.shape[0]
    assert A.shape[1] == (nq + 2 * nkv) * hd
    pos = np.ascontiguousarray(pos, np.int32)
    table = np.ascontiguousarray(table, np.float32)
    assert table.ndim == 3 and table.shape[1:] == (hd // 2, 2) and pos.shape == (M,)
    q = np.empty((M, nq, hd), np.uint16)
    k = np.empty((M, nkv, hd), np.uint16)
    v = np.empty((M, nkv, hd), np.uint16)
    rc = lib().orc_qkv_epilogue(M, nq, nkv, hd, _p(A, _c_f32p), float(alpha), _p(pos, _c_i32p),
                                _p(table, _c_f32p), table.shape[0], _p(q, _c_u16p), _p(k, _c_u16p), _p(v, _c_u16p))
    if rc:
        raise ValueError("position outside the rotary table")
    return q, k, v


@dataclass
class QkvWeights:
    """One layer's fused QKV projection: codes [(nq+2nkv)*hd, H] over the rows
    [Wq; Wk; Wv] with one per-tensor scale, the norm weight (unit when folded)
    and optional AdaRMSNorm modulation."""
    codes: np.ndarray
    s_w: float
    w_norm: np.ndarray
    nq: int
    nkv: int
    hd: int
    mod: Optional[tuple] = None

    @staticmethod
    def quantize(wq, wk, wv, w_norm, hd: int, norm_fuse: bool = False, mod=None) -> "QkvWeights":
        wq, wk, wv = _u16(wq), _u16(wk), _u16(wv)
        assert wq.shape[0] % hd == 0 and wk.shape == wv.shape and wk.shape[0] % hd == 0
        fused = np.ascontiguousarray(np.concatenate([wq, wk, wv], axis=0))
        w_norm = _u16(w_norm)
        if norm_fuse:
            codes, s = quant_tensor_fold(fused, w_norm)
            w_norm = np.full(w_norm.shape, ONES_BF16, np.uint16)
        else:
            codes, s = quant_tensor(fused)
        mod = None if mod is None else (_u16(mod[0]), _u16(mod[1]))
        return QkvWeights(codes, s, w_norm, wq.shape[0] // hd, wk.shape[0] // hd, hd, mod)


def qkv_block(r_prev, y_prev, qw: QkvWeights, eps: float, s_x: float, pos, table,
              nthreads: Optional[int] = None):
    """K1 then the fused QKV GEMM with the split + RoPE epilogue
    -> (r_out, xq, q, k, v)."""
    inv_x = np.float32(np.float32(1.0) / np.float32(s_x))
    r_out, _, xq = add_rmsnorm_quant(r_prev, y_prev, qw.w_norm, eps, float(inv_x), nthreads, mod=qw.mod)
    A = gemm_e4m3(xq, qw.codes, nthreads)
    alpha = np.float32(np.float32(s_x) * np.float32(qw.s_w))
    q, k, v = qkv_epilogue(A, float(alpha), qw.nq, qw.nkv, qw.hd, pos, table)
    return r_out, xq, q, k, v


def qkv_calibrate(batches, qw: QkvWeights, eps: float) -> float:
    """Static activation scale of the QKV GEMM input: amax of the normalised
    rows over the calibration batches (the measurement pass), then
    f32(amax / 448)."""
    amax = 0.0
    for r, y in batches:
        _, x, _ = add_rmsnorm_quant(r, y, qw.w_norm, eps, 1.0, mod=qw.mod)
        amax = max(amax, float(np.max(np.abs(x))))
    return scale_from_amax(amax)


# ---------------------------------------------------------------------------
# MXFP4 FFN variant (itsolotime article section 7.2: the NVFP4 encoder FFN
# with AWQ pre-scale and a 4-bit gated combine; here OCP MXFP4 blocks of 32
# with E8M0 scales).  Codes: E2M1 nibbles, element 2i in the low nibble of
# byte i; scales: E8M0 exponents e (X = 2^(e-127)), one per 32 elements.
# ---------------------------------------------------------------------------

def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, np.uint8)
    return np.vectorize(lambda x: lib().orc_e2m1_decode(int(x)), otypes=[np.float64])(c) if c.size else c.astype(float)


def e2m1_encode(v) -> np.ndarray:
    a = np.asarray(v, np.float64)
    return np.vectorize(lambda x: lib().orc_e2m1_encode(float(x)), otypes=[np.uint8])(a)


def mx_scale_exp(amax: float) -> int:
    return int(lib().orc_mx_scale_exp(float(amax)))


def mxfp4_quant_rows(v):
    """fp32 [rows, cols] (cols % 32 == 0) -> (codes [rows, cols/2], scales [rows, cols/32])."""
    v = np.ascontiguousarray(v, np.float32)
    rows, cols = v.shape
    assert cols % 32 == 0
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)
    lib().orc_mxfp4_quant_rows(_p(v, _c_f32p), rows, cols, _p(codes, _c_u8p), _p(scales, _c_u8p))
    return codes, scales


def mxfp4_quant_weight(w_bf16, colw_bf16=None):
    """bf16 [rows, cols] times the bf16 column factor (AWQ scale) -> MXFP4 along cols."""
    w = _u16(w_bf16)
    rows, cols = w.shape
    cw = None if colw_bf16 is None else _u16(colw_bf16)
    assert cw is None or cw.shape == (cols,)
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)
    rc = lib().orc_mxfp4_quant_weight(_p(w, _c_u16p), rows, cols, _p(cw, _c_u16p), _p(codes, _c_u8p),
                                      _p(scales, _c_u8p), default_threads())
    if rc:
        raise MemoryError("orc_mxfp4_quant_weight")
    return codes, scales


def mxfp4_gemm(a_codes, a_scales, b_codes, b_scales, nthreads: Optional[int] = None) -> np.ndarray:
    """f32(exact sum_k A[m][k] B[n][k]) for MXFP4 operands [M, K] and [N, K]."""
    ac, as_, bc, bs = (_u8(x) for x in (a_codes, a_scales, b_codes, b_scales))
    M, N, K = ac.shape[0], bc.shape[0], ac.shape[1] * 2
    assert bc.shape[1] * 2 == K and as_.shape == (M, K // 32) and bs.shape == (N, K // 32)
    out = np.empty((M, N), np.float32)
    rc = lib().orc_mxfp4_gemm(M, N, K, _p(ac, _c_u8p), _p(as_, _c_u8p), _p(bc, _c_u8p), _p(bs, _c_u8p),
                              _p(out, _c_f32p), nthreads or default_threads())
    if rc:
        raise ValueError("scale exponents spread beyond the exact accumulator")
    return out


@dataclass
class MxLayerWeights:
    """One layer in MXFP4: (codes, scales) of gate (None when non-gated), up and
    down, the norm weight, the AWQ reciprocal f32(1/s) [H] (None: no AWQ) and
    the optional AdaRMSNorm modulation."""
    g: Optional[tuple]
    u: tuple
    d: tuple
    w_norm: np.ndarray
    inv_awq: Optional[np.ndarray] = None
    mod: Optional[tuple] = None

    @staticmethod
    def quantize(w_gate, w_up, w_down, w_norm, awq=None, mod=None) -> "MxLayerWeights":
        """awq: bf16 [H] per-input-channel scale s (> 0): gate/up weights are
        quantised as f32(W[i][k] * s[k]) and the activations multiplied by
        f32(1 / s[k]); the down matrix is not scaled."""
        s = None if awq is None else _u16(awq)
        g = None if w_gate is None else mxfp4_quant_weight(w_gate, s)
        u = mxfp4_quant_weight(w_up, s)
        d = mxfp4_quant_weight(w_down, None)
        inv = None
        if s is not None:
            inv = (np.float32(1.0) / bf16_to_f32(s).astype(np.float32)).astype(np.float32)
        m = None if mod is None else (_u16(mod[0]), _u16(mod[1]))
        return MxLayerWeights(g, u, d, _u16(w_norm), inv, m)


def block_mxfp4(r_prev, y_prev, lw: MxLayerWeights, act: int, eps: float, nthreads: Optional[int] = None):
    """One MXFP4 block -> (r_out, (xq codes, scales), (hq codes, scales), y_out)."""
    r = _u16(r_prev)
    M, H = r.shape
    I = lw.u[0].shape[0]
    y = None if y_prev is None else _u16(y_prev)
    r_out = np.empty((M, H), np.uint16)
    xc = np.empty((M, H // 2), np.uint8)
    xs = np.empty((M, H // 32), np.uint8)
    hc = np.empty((M, I // 2), np.uint8)
    hs = np.empty((M, I // 32), np.uint8)
    y_out = np.empty((M, H), np.uint16)
    ms, mh = (None, None) if lw.mod is None else lw.mod
    gc, gs = (None, None) if lw.g is None else lw.g
    inv = None if lw.inv_awq is None else np.ascontiguousarray(lw.inv_awq, np.float32)
    rc = lib().orc_block_mxfp4(M, H, I, act, float(eps), _p(r, _c_u16p), _p(y, _c_u16p), _p(lw.w_norm, _c_u16p),
                               _p(ms, _c_u16p), _p(mh, _c_u16p), _p(inv, _c_f32p), _p(gc, _c_u8p), _p(gs, _c_u8p),
                               _p(lw.u[0], _c_u8p), _p(lw.u[1], _c_u8p), _p(lw.d[0], _c_u8p), _p(lw.d[1], _c_u8p),
                               _p(r_out, _c_u16p), _p(xc, _c_u8p), _p(xs, _c_u8p), _p(hc, _c_u8p), _p(hs, _c_u8p),
                               _p(y_out, _c_u16p), nthreads or default_threads())
    if rc:
        raise RuntimeError("orc_block_mxfp4 failed (%d)" % rc)
    return r_out, (xc, xs), (hc, hs), y_out


@dataclass
class MxChainResult:
    r: List[np.ndarray]
    y: List[Optional[np.ndarray]]
    xq: List[tuple]
    hq: List[tuple]


def run_chain_mxfp4(layers: Iterable[Callable[[], MxLayerWeights]], act: int, eps: float, r0, y0) -> MxChainResult:
    """Layer after layer in the pages' order (no calibration: the block scales
    are taken from the data as it flows)."""
    res = MxChainResult([_u16(r0)], [None if y0 is None else _u16(y0)], [], [])
    for get in layers:
        lw = get()
        r, xq, hq, y = block_mxfp4(res.r[-1], res.y[-1], lw, act, eps)
        res.r.append(r)
        res.y.append(y)
        res.xq.append(xq)
        res.hq.append(hq)
    return res
