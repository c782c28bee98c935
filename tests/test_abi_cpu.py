"""C-ABI checks that need no GPU: the library loads, exports every function
include/frt_ffn.h declares, and validates descriptors on the host."""
import os
import re

import pytest

from realtime_transformer_amd import _abi
from realtime_transformer_amd.configs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def _declared():
    names = set()
    for h in HEADERS:
        txt = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(frt_[a-z0-9_]+)\s*\(", txt))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    lib = _abi.load()
    names = _declared()
    assert "frt_ffn_plan_create" in names and "frt_graph_replay" in names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(_abi.EXPORTED)


def test_library_is_in_tree():
    assert os.path.dirname(_abi.lib_path()) == os.path.join(ROOT, "realtime_transformer_amd")


@pytest.mark.parametrize("bad", [
    dict(M=0), dict(L=0), dict(H=100), dict(I=200), dict(H=16384 + 128), dict(act=3),
    dict(eps=0.0), dict(eps=float("nan")), dict(flags=64), dict(flags=77), dict(flags=16 | 8), dict(flags=16 | 2),
    dict(M=1 << 20, H=4096, I=1024),
    dict(flags=32, H=384), dict(flags=32, I=1536 + 128), dict(flags=32 | 1), dict(flags=32 | 4),
    dict(flags=32 | 2), dict(flags=32 | 8), dict(device=-1)])
def test_bad_descriptors_rejected(bad):
    kw = dict(M=16, H=256, I=1024, L=1, act=0, eps=1e-6, device=0, flags=0)
    kw.update(bad)
    d = _abi.make_desc(**kw)
    with pytest.raises(_abi.FrtError) as e:
        _abi.frt_ffn_workspace_size(d)
    assert e.value.status == _abi.FRT_ERR_INVALID_ARG
    assert "invalid descriptor" in _abi.frt_last_error()


def test_workspace_sizes_cover_weights_and_slots():
    for c in CONFIGS.values():
        n = _abi.frt_ffn_workspace_size(_abi.make_desc(c.M, c.H, c.I, c.L, c.act))
        nw = (2 if c.gated else 1) * c.I * c.H + c.H * c.I
        slots = (2 * (c.L + 1) * c.M * c.H * 2) + c.L * c.M * (c.H + c.I)
        assert n >= c.L * nw + slots
        assert n < 1.2 * (c.L * nw + slots) + (1 << 30)


def test_plan_path_rejects_null_arguments():
    import ctypes
    lib = _abi.load()
    bits = ctypes.c_uint32(0)
    assert lib.frt_ffn_plan_path(None, ctypes.byref(bits)) == _abi.FRT_ERR_INVALID_ARG
    assert lib.frt_ffn_plan_path(None, None) == _abi.FRT_ERR_INVALID_ARG


def test_plan_create_rejects_null_workspace():
    d = _abi.make_desc(16, 256, 1024, 1, 0)
    with pytest.raises(_abi.FrtError) as e:
        _abi.frt_ffn_plan_create(d, 0, 1 << 20)
    assert e.value.status == _abi.FRT_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [
    dict(M=0), dict(H=100), dict(H=16384 + 128), dict(nq=0), dict(nkv=0), dict(hd=48), dict(hd=16), dict(hd=544),
    dict(max_pos=0), dict(eps=0.0), dict(rope_base=1.0), dict(rope_base=float("inf")), dict(flags=1), dict(flags=2),
    dict(flags=8 | 16), dict(device=-1), dict(M=1 << 20, H=4096)])
def test_bad_qkv_descriptors_rejected(bad):
    kw = dict(M=4, H=256, nq=2, nkv=1, hd=64, max_pos=32, eps=1e-6, rope_base=1e4, device=0, flags=0)
    kw.update(bad)
    with pytest.raises(_abi.FrtError) as e:
        _abi.frt_qkv_workspace_size(_abi.make_qkv_desc(**kw))
    assert e.value.status == _abi.FRT_ERR_INVALID_ARG


def test_qkv_workspace_covers_weights_table_and_slots():
    from realtime_transformer_amd.configs import QKV_CONFIGS
    for c in QKV_CONFIGS.values():
        n = _abi.frt_qkv_workspace_size(_abi.make_qkv_desc(c.M, c.H, c.nq, c.nkv, c.hd, c.max_pos, c.eps, c.rope_base))
        need = c.N * c.H + c.max_pos * c.hd * 4 + c.M * c.H * (2 + 2 + 2 + 1) + 2 * c.M * c.N
        assert need <= n < 1.3 * need + (1 << 24)
    for flags in (8, 16):
        assert _abi.frt_qkv_workspace_size(_abi.make_qkv_desc(4, 256, 2, 1, 64, 32, flags=flags)) > 0


def test_mxfp4_descriptors_accepted():
    for kw in (dict(M=1, H=512, I=1024), dict(M=64, H=1024, I=4096, flags_extra=16)):
        extra = kw.pop("flags_extra", 0)
        n = _abi.frt_ffn_workspace_size(_abi.make_desc(kw["M"], kw["H"], kw["I"], 2, 0, flags=32 | extra))
        fp8 = _abi.frt_ffn_workspace_size(_abi.make_desc(kw["M"], kw["H"], kw["I"], 2, 0))
        assert 0 < n < fp8  # 4-bit weights take about half the bytes
