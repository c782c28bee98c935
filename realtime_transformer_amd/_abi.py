"""ctypes binding of libfrt (include/frt_ffn.h): argument marshalling only.

Every function keeps the C name, takes plain ints for device pointers and
streams, converts the status code into FrtError, and does nothing else; all
work happens in the HIP library.  There is no fallback: if libfrt.so cannot be
loaded the import-time call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import build as _build

FRT_OK = 0
FRT_ERR_INVALID_ARG = 1
FRT_ERR_HIP = 2
FRT_ERR_STATE = 3
FRT_ERR_UNSUPPORTED = 4
FRT_ERR_WORKSPACE = 5

FRT_ACT_GEGLU_TANH = 0
FRT_ACT_SWIGLU = 1
FRT_ACT_GELU_TANH = 2

FRT_FLAG_FP8_MFMA_DOWN = 1
FRT_FLAG_FUSED_NORM = 2
FRT_FLAG_FP8_MFMA_GATEUP = 4
FRT_FLAG_NORM_FUSE = 8
FRT_FLAG_ADA_NORM = 16
FRT_FLAG_MXFP4 = 32

FRT_PATH_GEMV = 1
FRT_PATH_NORM_SPLIT = 2
FRT_PATH_DOWN_WHOLE_COLUMN = 4
FRT_PATH_DOWN_SPLIT_K = 8
FRT_PATH_GATEUP_OCTETS = 16

_STATUS_NAMES = {0: "FRT_OK", 1: "FRT_ERR_INVALID_ARG", 2: "FRT_ERR_HIP", 3: "FRT_ERR_STATE",
                 4: "FRT_ERR_UNSUPPORTED", 5: "FRT_ERR_WORKSPACE"}

EXPORTED = [
    "frt_ffn_workspace_size", "frt_ffn_plan_create", "frt_ffn_plan_destroy", "frt_quant_weights",
    "frt_export_weight_codes", "frt_calibrate", "frt_get_scales", "frt_set_act_scales",
    "frt_ffn_io_get", "frt_ffn_forward_range", "frt_ffn_forward", "frt_graph_capture",
    "frt_graph_replay", "frt_ffn_forward_profiled", "frt_ffn_time_kernel", "frt_e4m3_encode_f32",
    "frt_last_error", "frt_export_mxfp4_weights", "frt_set_awq", "frt_ffn_forward_range_static_scratch",
    "frt_ffn_plan_path", "frt_ffn_desc_path",
    # attention input (include/frt_qkv.h)
    "frt_qkv_workspace_size", "frt_qkv_plan_create", "frt_qkv_plan_destroy", "frt_qkv_quant_weights",
    "frt_qkv_export_weight_codes", "frt_qkv_calibrate", "frt_qkv_get_scales", "frt_qkv_set_act_scale",
    "frt_qkv_set_positions", "frt_qkv_io_get", "frt_qkv_forward", "frt_qkv_time_kernel",
    "frt_qkv_graph_capture", "frt_qkv_graph_replay",
]


class FrtError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (_STATUS_NAMES.get(status, str(status)), msg))
        self.status = status


class frt_ffn_desc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("L", ctypes.c_int32), ("act", ctypes.c_int32), ("eps", ctypes.c_float),
                ("device", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class frt_ffn_io(ctypes.Structure):
    _fields_ = [("r_slots", ctypes.c_void_p), ("y_slots", ctypes.c_void_p),
                ("xq_slots", ctypes.c_void_p), ("hq_slots", ctypes.c_void_p),
                ("z_out", ctypes.c_void_p), ("stride_rh", ctypes.c_size_t),
                ("stride_xq", ctypes.c_size_t), ("stride_hq", ctypes.c_size_t),
                ("mod_slots", ctypes.c_void_p), ("stride_mod", ctypes.c_size_t)]


class frt_qkv_desc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int32), ("H", ctypes.c_int32), ("nq", ctypes.c_int32),
                ("nkv", ctypes.c_int32), ("hd", ctypes.c_int32), ("max_pos", ctypes.c_int32),
                ("eps", ctypes.c_float), ("rope_base", ctypes.c_float), ("device", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class frt_qkv_io(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("r_in", "y_in", "pos", "mod", "r_out", "xq", "q", "k", "v", "rope")]


_lib = None


def lib_path() -> str:
    return _build.LIB


def load(build_if_missing: bool = True):
    """Load libfrt.so (building it first only when no library exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        if not build_if_missing:
            raise FrtError(FRT_ERR_UNSUPPORTED, "libfrt.so is not built")
        _build.build(force=True)
    L = ctypes.CDLL(_build.LIB)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "frt_ffn_workspace_size": [ctypes.POINTER(frt_ffn_desc), ctypes.POINTER(sz)],
        "frt_ffn_plan_create": [ctypes.POINTER(frt_ffn_desc), vp, sz, ctypes.POINTER(vp)],
        "frt_ffn_plan_destroy": [vp],
        "frt_quant_weights": [vp, i32, vp, vp, vp, vp, vp],
        "frt_export_weight_codes": [vp, i32, i32, vp],
        "frt_calibrate": [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32, i32, i32, vp],
        "frt_get_scales": [vp, ctypes.POINTER(ctypes.c_float)],
        "frt_set_act_scales": [vp, ctypes.POINTER(ctypes.c_float)],
        "frt_ffn_io_get": [vp, ctypes.POINTER(frt_ffn_io)],
        "frt_ffn_plan_path": [vp, ctypes.POINTER(ctypes.c_uint32)],
        "frt_ffn_desc_path": [ctypes.POINTER(frt_ffn_desc), ctypes.POINTER(ctypes.c_uint32)],
        "frt_ffn_forward_range": [vp, i32, i32, vp],
        "frt_ffn_forward_range_static_scratch": [vp, i32, i32, vp],
        "frt_ffn_forward": [vp, vp],
        "frt_graph_capture": [vp, vp],
        "frt_graph_replay": [vp, vp],
        "frt_ffn_forward_profiled": [vp, vp, ctypes.POINTER(ctypes.c_float)],
        "frt_ffn_time_kernel": [vp, i32, i32, vp, ctypes.POINTER(ctypes.c_float)],
        "frt_e4m3_encode_f32": [vp, vp, ctypes.c_int64, vp],
        "frt_export_mxfp4_weights": [vp, i32, i32, vp, vp],
        "frt_set_awq": [vp, i32, vp, vp],
        "frt_qkv_workspace_size": [ctypes.POINTER(frt_qkv_desc), ctypes.POINTER(sz)],
        "frt_qkv_plan_create": [ctypes.POINTER(frt_qkv_desc), vp, sz, ctypes.POINTER(vp)],
        "frt_qkv_plan_destroy": [vp],
        "frt_qkv_quant_weights": [vp, vp, vp, vp, vp, vp],
        "frt_qkv_export_weight_codes": [vp, vp],
        "frt_qkv_calibrate": [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32, vp],
        "frt_qkv_get_scales": [vp, ctypes.POINTER(ctypes.c_float)],
        "frt_qkv_set_act_scale": [vp, ctypes.c_float],
        "frt_qkv_set_positions": [vp, ctypes.POINTER(ctypes.c_int32), vp],
        "frt_qkv_io_get": [vp, ctypes.POINTER(frt_qkv_io)],
        "frt_qkv_forward": [vp, vp],
        "frt_qkv_time_kernel": [vp, i32, i32, vp, ctypes.POINTER(ctypes.c_float)],
        "frt_qkv_graph_capture": [vp, vp],
        "frt_qkv_graph_replay": [vp, vp],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.frt_last_error.argtypes = []
    L.frt_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != FRT_OK:
        raise FrtError(status, load().frt_last_error().decode(errors="replace"))


def make_desc(M: int, H: int, I: int, L: int, act: int, eps: float = 1e-6, device: int = 0,
              flags: int = 0) -> frt_ffn_desc:
    return frt_ffn_desc(M, H, I, L, act, eps, device, flags)


def frt_ffn_workspace_size(desc: frt_ffn_desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load().frt_ffn_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def frt_ffn_plan_create(desc: frt_ffn_desc, d_workspace: int, nbytes: int) -> int:
    out = ctypes.c_void_p(None)
    _check(load().frt_ffn_plan_create(ctypes.byref(desc), ctypes.c_void_p(d_workspace), nbytes,
                                      ctypes.byref(out)))
    return out.value


def frt_ffn_plan_destroy(plan: Optional[int]) -> None:
    _check(load().frt_ffn_plan_destroy(ctypes.c_void_p(plan)))


def frt_quant_weights(plan: int, layer: int, d_w_gate: Optional[int], d_w_up: int, d_w_down: int,
                      d_norm_w: int, stream: int) -> None:
    _check(load().frt_quant_weights(plan, layer, d_w_gate, d_w_up, d_w_down, d_norm_w, stream))


def frt_export_weight_codes(plan: int, layer: int, which: int, rows: int, cols: int) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint8)
    _check(load().frt_export_weight_codes(plan, layer, which, out.ctypes.data_as(ctypes.c_void_p)))
    return out


def frt_calibrate(plan: int, d_r_batches: Sequence[int], d_y_batches: Optional[Sequence[int]],
                  rows: int, layer_begin: int, layer_end: int, stream: int) -> None:
    n = len(d_r_batches)
    rb = (ctypes.c_void_p * n)(*d_r_batches)
    yb = None if d_y_batches is None else (ctypes.c_void_p * n)(*d_y_batches)
    _check(load().frt_calibrate(plan, rb, yb, n, rows, layer_begin, layer_end, stream))


def frt_get_scales(plan: int, L: int) -> np.ndarray:
    out = np.zeros((L, 5), dtype=np.float32)
    _check(load().frt_get_scales(plan, out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
    return out


def frt_set_act_scales(plan: int, scales) -> None:
    a = np.ascontiguousarray(np.asarray(scales, dtype=np.float32))
    _check(load().frt_set_act_scales(plan, a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))


def frt_ffn_plan_path(plan: int) -> int:
    bits = ctypes.c_uint32(0)
    _check(load().frt_ffn_plan_path(plan, ctypes.byref(bits)))
    return int(bits.value)


def frt_ffn_desc_path(desc: frt_ffn_desc) -> int:
    """FRT_PATH_* bits of a plan with this descriptor (host only)."""
    bits = ctypes.c_uint32(0)
    _check(load().frt_ffn_desc_path(ctypes.byref(desc), ctypes.byref(bits)))
    return int(bits.value)


def frt_ffn_io_get(plan: int) -> frt_ffn_io:
    io = frt_ffn_io()
    _check(load().frt_ffn_io_get(plan, ctypes.byref(io)))
    return io


def frt_ffn_forward_range(plan: int, layer_begin: int, layer_end: int, stream: int) -> None:
    _check(load().frt_ffn_forward_range(plan, layer_begin, layer_end, stream))


def frt_ffn_forward_range_static_scratch(plan: int, layer_begin: int, layer_end: int, stream: int) -> None:
    _check(load().frt_ffn_forward_range_static_scratch(plan, layer_begin, layer_end, stream))


def frt_ffn_forward(plan: int, stream: int) -> None:
    _check(load().frt_ffn_forward(plan, stream))


def frt_graph_capture(plan: int, stream: int) -> None:
    _check(load().frt_graph_capture(plan, stream))


def frt_graph_replay(plan: int, stream: int) -> None:
    _check(load().frt_graph_replay(plan, stream))


def frt_ffn_forward_profiled(plan: int, stream: int, L: int) -> np.ndarray:
    out = np.zeros((L, 3), dtype=np.float32)
    _check(load().frt_ffn_forward_profiled(plan, stream, out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
    return out


def frt_ffn_time_kernel(plan: int, which: int, reps: int, stream: int) -> float:
    out = ctypes.c_float(0.0)
    _check(load().frt_ffn_time_kernel(plan, which, reps, stream, ctypes.byref(out)))
    return float(out.value)


def frt_e4m3_encode_f32(d_in: int, d_out: int, n: int, stream: int) -> None:
    _check(load().frt_e4m3_encode_f32(d_in, d_out, n, stream))


def frt_last_error() -> str:
    return load().frt_last_error().decode(errors="replace")


# ---------------------------------------------------------------------------
# attention input (include/frt_qkv.h)
# ---------------------------------------------------------------------------

def make_qkv_desc(M: int, H: int, nq: int, nkv: int, hd: int, max_pos: int, eps: float = 1e-6,
                  rope_base: float = 10000.0, device: int = 0, flags: int = 0) -> frt_qkv_desc:
    return frt_qkv_desc(M, H, nq, nkv, hd, max_pos, eps, rope_base, device, flags)


def frt_qkv_workspace_size(desc: frt_qkv_desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load().frt_qkv_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def frt_qkv_plan_create(desc: frt_qkv_desc, d_workspace: int, nbytes: int) -> int:
    out = ctypes.c_void_p(None)
    _check(load().frt_qkv_plan_create(ctypes.byref(desc), ctypes.c_void_p(d_workspace), nbytes, ctypes.byref(out)))
    return out.value


def frt_qkv_plan_destroy(plan: Optional[int]) -> None:
    _check(load().frt_qkv_plan_destroy(ctypes.c_void_p(plan)))


def frt_qkv_quant_weights(plan: int, d_wq: int, d_wk: int, d_wv: int, d_norm_w: int, stream: int) -> None:
    _check(load().frt_qkv_quant_weights(plan, d_wq, d_wk, d_wv, d_norm_w, stream))


def frt_qkv_export_weight_codes(plan: int, rows: int, cols: int) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint8)
    _check(load().frt_qkv_export_weight_codes(plan, out.ctypes.data_as(ctypes.c_void_p)))
    return out


def frt_qkv_calibrate(plan: int, d_r_batches: Sequence[int], d_y_batches: Optional[Sequence[int]], rows: int,
                      stream: int) -> None:
    n = len(d_r_batches)
    rb = (ctypes.c_void_p * n)(*d_r_batches)
    yb = None if d_y_batches is None else (ctypes.c_void_p * n)(*d_y_batches)
    _check(load().frt_qkv_calibrate(plan, rb, yb, n, rows, stream))


def frt_qkv_get_scales(plan: int) -> np.ndarray:
    out = np.zeros(2, dtype=np.float32)
    _check(load().frt_qkv_get_scales(plan, out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
    return out


def frt_qkv_set_act_scale(plan: int, s_x: float) -> None:
    _check(load().frt_qkv_set_act_scale(plan, float(s_x)))


def frt_qkv_set_positions(plan: int, pos, stream: int) -> None:
    a = np.ascontiguousarray(np.asarray(pos, dtype=np.int32))
    _check(load().frt_qkv_set_positions(plan, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), stream))


def frt_qkv_io_get(plan: int) -> frt_qkv_io:
    io = frt_qkv_io()
    _check(load().frt_qkv_io_get(plan, ctypes.byref(io)))
    return io


def frt_qkv_forward(plan: int, stream: int) -> None:
    _check(load().frt_qkv_forward(plan, stream))


def frt_qkv_time_kernel(plan: int, which: int, reps: int, stream: int) -> float:
    us = ctypes.c_float(0.0)
    _check(load().frt_qkv_time_kernel(plan, which, reps, stream, ctypes.byref(us)))
    return us.value


def frt_qkv_graph_capture(plan: int, stream: int) -> None:
    _check(load().frt_qkv_graph_capture(plan, stream))


def frt_qkv_graph_replay(plan: int, stream: int) -> None:
    _check(load().frt_qkv_graph_replay(plan, stream))


def frt_export_mxfp4_weights(plan: int, layer: int, which: int, rows: int, cols: int):
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    exps = np.empty((rows, cols // 32), dtype=np.uint8)
    _check(load().frt_export_mxfp4_weights(plan, layer, which, codes.ctypes.data_as(ctypes.c_void_p),
                                           exps.ctypes.data_as(ctypes.c_void_p)))
    return codes, exps


def frt_set_awq(plan: int, layer: int, d_awq: int, stream: int) -> None:
    _check(load().frt_set_awq(plan, layer, d_awq, stream))
