"""C-ABI checks that need no GPU: the library loads, exports every function
include/frt_ffn.h declares, and validates descriptors on the host."""
import os
import re

import pytest

from realtime_transformer_amd import _abi
from realtime_transformer_amd.configs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "frt_ffn.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(frt_[a-z0-9_]+)\s*\(", txt)))


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
    dict(eps=0.0), dict(eps=float("nan")), dict(flags=32), dict(flags=45), dict(flags=16 | 8), dict(flags=16 | 2),
    dict(device=-1)])
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


def test_plan_create_rejects_null_workspace():
    d = _abi.make_desc(16, 256, 1024, 1, 0)
    with pytest.raises(_abi.FrtError) as e:
        _abi.frt_ffn_plan_create(d, 0, 1 << 20)
    assert e.value.status == _abi.FRT_ERR_INVALID_ARG
