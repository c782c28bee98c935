"""Kernel-path selection on the host (frt_ffn_desc_path: the FRT_PATH_* bits
a plan from a descriptor would have, no device call): which decode layer
the plan runs for each shape, format, flag and environment override."""
import ctypes

import pytest

from realtime_transformer_amd import _abi
from realtime_transformer_amd.configs import ACT_GEGLU_TANH, ACT_SWIGLU, ACT_GELU_TANH

GEMV = _abi.FRT_PATH_GEMV
SPLIT = _abi.FRT_PATH_NORM_SPLIT
WHOLE = _abi.FRT_PATH_DOWN_WHOLE_COLUMN
SPLITK = _abi.FRT_PATH_DOWN_SPLIT_K
OCT = _abi.FRT_PATH_GATEUP_OCTETS
MX = _abi.FRT_FLAG_MXFP4

# the dense-LLM decode shape (H = 5120, I = 17408)
H, I = 5120, 17408


def _path(M, h, i, act=ACT_SWIGLU, flags=0, L=2):
    return _abi.frt_ffn_desc_path(_abi.make_desc(M, h, i, L, act, flags=flags))


@pytest.fixture(autouse=True)
def _clean_env(monkeypatch):
    for k in ("FRT_DOWN_QUAD", "FRT_GATEUP_OCT", "FRT_NORM_SPLIT", "FRT_GEMV_DOWN_SPLIT", "FRT_GEMV_WAVES_GATEUP",
              "FRT_GEMV_WAVES_GATEUP_MX", "FRT_GEMV_MT_MAX_M"):
        monkeypatch.delenv(k, raising=False)


def test_decode_m1_is_two_kernels_per_layer():
    # split norm, octet gate/up, whole-column down: no split-K partials
    assert _path(1, H, I) == GEMV | SPLIT | WHOLE | OCT
    assert _path(3, H, I, ACT_GEGLU_TANH) == GEMV | SPLIT | WHOLE | OCT
    assert _path(4, 2048, 8192, ACT_GEGLU_TANH) == GEMV | SPLIT | WHOLE | OCT
    # the split norm holds the rows' codes in LDS (16 KiB): M = 4 at H = 5120
    # takes the one-kernel norm and the split-K down GEMV
    assert _path(4, H, I) == GEMV | SPLITK
    # tanh-GELU has no gate: no octets, still whole columns
    assert _path(1, H, I, ACT_GELU_TANH) == GEMV | SPLIT | WHOLE


def test_decode_overrides(monkeypatch):
    monkeypatch.setenv("FRT_DOWN_QUAD", "0")
    assert _path(1, H, I) == GEMV | SPLIT | SPLITK | OCT
    monkeypatch.setenv("FRT_GATEUP_OCT", "0")
    assert _path(1, H, I) == GEMV | SPLIT | SPLITK
    monkeypatch.delenv("FRT_DOWN_QUAD")
    assert _path(1, H, I) == GEMV | SPLIT | WHOLE
    monkeypatch.setenv("FRT_NORM_SPLIT", "0")  # the one-kernel norm: the down GEMV splits K again
    assert _path(1, H, I) == GEMV | SPLITK


def test_whole_column_needs_at_most_four_rows():
    b = _path(5, 1024, 4096)
    assert b & GEMV and b & SPLIT and b & OCT and not b & WHOLE


def test_fused_and_modulated_norms_keep_the_split_k_down():
    for f in (_abi.FRT_FLAG_FUSED_NORM, _abi.FRT_FLAG_ADA_NORM):
        b = _path(1, H, I, flags=f)
        assert b & GEMV and not b & (SPLIT | WHOLE | OCT), (f, b)


def test_prefill_sizes_leave_the_gemv_path():
    for M in (50, 788, 4096):
        b = _path(M, 2048, 16384, ACT_GEGLU_TANH)
        assert not b & (GEMV | SPLIT | WHOLE | OCT), (M, b)


def test_mxfp4_decode_paths(monkeypatch):
    assert _path(1, H, I, flags=MX) == GEMV | SPLIT | WHOLE
    assert _path(2, 512, 2048, ACT_GEGLU_TANH, flags=MX) == GEMV | SPLIT | WHOLE
    b = _path(7, 512, 2048, ACT_GEGLU_TANH, flags=MX)
    assert b & GEMV and b & SPLIT and not b & (WHOLE | OCT)
    b = _path(300, 512, 2048, flags=MX)
    assert not b & (GEMV | SPLIT | WHOLE | OCT)
    monkeypatch.setenv("FRT_DOWN_QUAD", "0")
    assert _path(1, H, I, flags=MX) == GEMV | SPLIT | SPLITK


def test_mxfp4_overrides_beyond_the_kernels_are_not_taken(monkeypatch):
    # eight gate/up waves do not fit four row tiles (M = 50): the plan keeps
    # its own choice; a split beyond the 512-value quads is clamped, so the
    # descriptor stays valid either way
    monkeypatch.setenv("FRT_GEMV_WAVES_GATEUP_MX", "8")
    assert _path(50, 1024, 4096, ACT_GEGLU_TANH, flags=MX) & SPLITK
    monkeypatch.setenv("FRT_GEMV_DOWN_SPLIT", "64")
    assert _path(7, 512, 2048, ACT_GEGLU_TANH, flags=MX) & SPLITK


def test_desc_path_rejects_null_and_invalid():
    lib = _abi.load()
    bits = ctypes.c_uint32(0)
    d = _abi.make_desc(1, H, I, 2, ACT_SWIGLU)
    assert lib.frt_ffn_desc_path(None, ctypes.byref(bits)) == _abi.FRT_ERR_INVALID_ARG
    assert lib.frt_ffn_desc_path(ctypes.byref(d), None) == _abi.FRT_ERR_INVALID_ARG
    bad = _abi.make_desc(1, 100, I, 2, ACT_SWIGLU)  # H not a multiple of the K block
    assert lib.frt_ffn_desc_path(ctypes.byref(bad), ctypes.byref(bits)) == _abi.FRT_ERR_INVALID_ARG
