"""Pins of the oracle's E4M3 and bf16 codecs against the OCP table, IEEE
rounding rules and torch's own converters (library cross-checks)."""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            rows.append(parts)
    return rows


def test_ocp_table_values():
    for code, value, *_ in _read_table("e4m3_ocp_table.txt"):
        c = int(code, 16)
        got = float(oracle.e4m3_decode(np.array([c], np.uint8))[0])
        if value == "nan":
            assert math.isnan(got), code
        elif value == "-0":
            assert got == 0.0 and math.copysign(1.0, got) < 0, code
        else:
            assert got == float(value), (code, got, value)
            if value != "0":
                assert int(oracle.e4m3_encode(np.array([float(value)], np.float32))[0]) == c


def test_rounding_cases():
    for inp, code, *_ in _read_table("e4m3_rounding.txt"):
        x = np.array([float(inp)], np.float32)
        assert int(oracle.e4m3_encode(x)[0]) == int(code, 16), (inp, code)


def test_exhaustive_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert len(codes) == 254
    vals = oracle.e4m3_decode(codes)
    back = oracle.e4m3_encode(vals.astype(np.float32))
    assert np.array_equal(back, codes)
    # decoded values are strictly increasing over positive codes 0..0x7e
    pos = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    assert pos[-1] == 448.0
    nan_codes = oracle.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))
    assert np.all(np.isnan(nan_codes))


def test_nan_maps_to_nan_code():
    out = oracle.e4m3_encode(np.array([np.nan, -np.nan], np.float32))
    assert set((out & 0x7F).tolist()) == {0x7F}


def _boundary_values():
    pos = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    base = np.concatenate([pos, mids, [448, 460, 464, 470, 480, 500, 1e6]]).astype(np.float32)
    vals = [base]
    up, dn = base.copy(), base.copy()
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        vals += [up, dn]
    v = np.concatenate(vals)
    return np.concatenate([v, -v])


def test_matches_torch_float8_with_clamp():
    # torch's CPU float8_e4m3fn cast rounds to nearest even but turns values
    # beyond 464 into NaN; clamping to +-448 first gives the saturating
    # quantiser, which must agree with the oracle code for code.
    rng = np.random.default_rng(11)
    n = 4_000_000
    r = (rng.standard_normal(n) * np.exp(rng.uniform(-14, 7, n))).astype(np.float32)
    x = np.concatenate([_boundary_values(), r]).astype(np.float32)
    ref = torch.from_numpy(x).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(x)
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, (x[bad[:5]], ref[bad[:5]], got[bad[:5]])


def test_saturation_invariant_on_large_values():
    x = np.array([448.0, 449.0, 1e3, 1e38, np.inf, -np.inf, -1e5], np.float32)
    c = oracle.e4m3_encode(x)
    assert np.all((c & 0x7F) == 0x7E)
    assert np.all(np.abs(oracle.e4m3_decode(c)) <= 448)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(2_000_000) * np.exp(rng.uniform(-30, 30, 2_000_000))).astype(np.float32)
    ties = np.array([1.00390625, 1.01171875, -1.00390625, 3.0e-39, 65504.0, 1e38], np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(x)
    assert np.array_equal(ref, got)
    # ties to even
    assert oracle.bf16_to_f32(oracle.bf16_round(np.float32(1.00390625)))[()] == 1.0
    assert oracle.bf16_to_f32(oracle.bf16_round(np.float32(1.01171875)))[()] == 1.015625


def test_bf16_widen_is_exact():
    b = np.arange(0, 1 << 16, dtype=np.uint16)
    f = oracle.bf16_to_f32(b)
    ok = np.isfinite(f)
    assert np.array_equal(oracle.bf16_round(f[ok]), b[ok])
