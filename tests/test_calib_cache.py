"""Host-side checks of the calibration cache (key, file name, JSON round
trip, validation, miss/hit flow), against a stand-in plan object."""
import json
import os

import numpy as np
import pytest

from realtime_transformer_amd import calib_cache as cc


def _layers(seed, L=3, H=128, I=256, gated=True):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(L):
        g = rng.integers(0, 1 << 16, (I, H), dtype=np.uint16) if gated else None
        out.append((g, rng.integers(0, 1 << 16, (I, H), dtype=np.uint16),
                    rng.integers(0, 1 << 16, (H, I), dtype=np.uint16), rng.integers(0, 1 << 16, H, dtype=np.uint16)))
    return out


def _hash(layers, **kw):
    a = dict(H=128, I=256, L=len(layers), act=0, eps=1e-6, flags=0)
    a.update(kw)
    return cc.ckpt_hash(a["H"], a["I"], a["L"], a["act"], a["eps"], layers, a["flags"])


def test_hash_is_deterministic_and_sensitive_to_every_tensor():
    ls = _layers(1)
    h0 = _hash(ls)
    assert h0 == _hash(_layers(1)) and len(h0) == 16
    for li in range(3):
        for ti in range(4):
            mod = [list(t) for t in ls]
            t = mod[li][ti].copy()
            t.reshape(-1)[7] ^= 1  # one bit of one bf16 value
            mod[li][ti] = t
            assert _hash(mod) != h0, (li, ti)


def test_hash_covers_layer_order_shapes_and_scale_settings():
    ls = _layers(2)
    h0 = _hash(ls)
    assert _hash(ls[::-1]) != h0
    assert _hash(ls, act=1) != h0
    assert _hash(ls, eps=1e-5) != h0
    assert _hash(ls, flags=8) != h0 and _hash(ls, flags=16) != h0
    # kernel-choice flags do not change the scales, so they do not change the key
    assert _hash(ls, flags=1 | 2 | 4) == h0
    # same bytes, other shape
    reshaped = [(g.reshape(128, 256), u, d, n) for g, u, d, n in ls]
    assert _hash(reshaped) != h0
    # gated vs ungated (absent gate)
    ung = [(None, u, d, n) for _, u, d, n in ls]
    assert _hash(ung) != h0


def test_file_name_follows_hash_and_sequence_length(tmp_path):
    p = cc.cache_path("0123abcd", 788, str(tmp_path))
    assert os.path.basename(p) == "0123abcd_Se788.json"
    assert cc.cache_path("0123abcd", 50, str(tmp_path)) != p
    with pytest.raises(ValueError):
        cc.cache_path("../x", 1, str(tmp_path))
    with pytest.raises(ValueError):
        cc.cache_path("ab", 0, str(tmp_path))


def test_default_dir_honours_environment(monkeypatch, tmp_path):
    monkeypatch.setenv(cc.ENV_DIR, str(tmp_path))
    assert cc.default_dir() == str(tmp_path)
    monkeypatch.delenv(cc.ENV_DIR)
    assert cc.default_dir().endswith(os.path.join(".realtime_transformer_amd", "calibration"))


def _awkward_f32(n, seed):
    rng = np.random.default_rng(seed)
    v = rng.uniform(1e-6, 10.0, n).astype(np.float32)
    v[0] = np.float32(1.0) / np.float32(3.0)
    v[1] = np.nextafter(np.float32(1.0), np.float32(2.0))
    v[2] = np.float32(np.finfo(np.float32).tiny) * 3  # small normal
    v[3] = np.float32(448.0) / np.float32(7.0)
    return v


def test_round_trip_is_bit_exact_and_keeps_extra(tmp_path):
    L = 9
    rec = cc.CalibRecord("feedbeef", 50, _awkward_f32(L, 1), _awkward_f32(L, 2),
                         _awkward_f32(3 * L, 3).reshape(L, 3), {"note": "x", "awq": [1, 2]})
    p = cc.save(cc.cache_path("feedbeef", 50, str(tmp_path)), rec)
    got = cc.load(p, expect_ckpt="feedbeef", expect_seq=50, expect_layers=L)
    assert got.s_x.dtype == np.float32
    assert np.array_equal(got.s_x.view(np.uint32), rec.s_x.view(np.uint32))
    assert np.array_equal(got.s_h.view(np.uint32), rec.s_h.view(np.uint32))
    assert np.array_equal(got.s_w.view(np.uint32), rec.s_w.view(np.uint32))
    assert got.extra == {"note": "x", "awq": [1, 2]}
    assert [f for f in os.listdir(tmp_path) if f.startswith(".calib-")] == []


def _write(tmp_path, doc):
    p = str(tmp_path / "x_Se1.json")
    with open(p, "w") as f:
        f.write(doc if isinstance(doc, str) else json.dumps(doc))
    return p


GOOD = {"format": 1, "ckpt_hash": "x", "seq": 1, "layers": 2, "s_x": [0.5, 0.25], "s_h": [1.0, 2.0],
        "s_w": None, "extra": {}}


@pytest.mark.parametrize("bad", [
    {"format": 2}, {"s_x": [0.5]}, {"layers": 3}, {"s_x": [0.5, -1.0]}, {"s_h": [0.0, 1.0]},
    {"s_x": [0.1, 0.25]},  # 0.1 is not a float32 value
    {"s_x": []}, {"s_x": "0.5"}, {"extra": [1]}])
def test_load_rejects_malformed_files(tmp_path, bad):
    doc = dict(GOOD)
    doc.update(bad)
    with pytest.raises(ValueError):
        cc.load(_write(tmp_path, doc))


def test_load_rejects_non_finite_and_mismatches(tmp_path):
    txt = json.dumps(GOOD).replace("0.25", "NaN")
    with pytest.raises(ValueError):
        cc.load(_write(tmp_path, txt))
    p = _write(tmp_path, GOOD)
    cc.load(p)
    with pytest.raises(ValueError):
        cc.load(p, expect_ckpt="y")
    with pytest.raises(ValueError):
        cc.load(p, expect_seq=2)
    with pytest.raises(ValueError):
        cc.load(p, expect_layers=3)


def test_save_refuses_invalid_scales(tmp_path):
    with pytest.raises(ValueError):
        cc.save(str(tmp_path / "a.json"), cc.CalibRecord("a", 1, np.array([np.inf], np.float32),
                                                         np.array([1.0], np.float32)))
    with pytest.raises(ValueError):
        cc.save(str(tmp_path / "a.json"), cc.CalibRecord("a", 1, np.array([1.0, 2.0], np.float32),
                                                         np.array([1.0], np.float32)))
    assert not os.path.exists(tmp_path / "a.json")


class _StubPlan:
    """Stand-in for FFNPlan with the three calls the cache uses."""

    def __init__(self, M, L, seed):
        self.M, self.L = M, L
        self.sc = np.zeros((L, 5), np.float32)
        self.measured = _awkward_f32(2 * L, seed).reshape(L, 2)
        self.calls = []

    def calibrate(self, batches):
        self.calls.append("calibrate")
        self.sc[:, 0], self.sc[:, 3] = self.measured[:, 0], self.measured[:, 1]
        self.sc[:, [1, 2, 4]] = 0.01

    def scales(self):
        return self.sc.copy()

    def set_act_scales(self, s_x, s_h):
        self.calls.append("set")
        self.sc[:, 0], self.sc[:, 3] = s_x, s_h


def test_miss_measures_and_saves_then_hit_installs_the_same_bits(tmp_path):
    a = _StubPlan(16, 4, 5)
    assert cc.calibrate_cached(a, "abc123", ["batch"], root=str(tmp_path), extra={"k": 1}) is False
    assert a.calls == ["calibrate"]
    assert os.path.exists(tmp_path / "abc123_Se16.json")
    b = _StubPlan(16, 4, 99)  # would measure other values
    assert cc.calibrate_cached(b, "abc123", None, root=str(tmp_path)) is True
    assert b.calls == ["set"]
    assert np.array_equal(b.sc[:, [0, 3]].view(np.uint32), a.sc[:, [0, 3]].view(np.uint32))
    assert cc.load(str(tmp_path / "abc123_Se16.json")).extra == {"k": 1}
    # another M is another file: a miss
    c = _StubPlan(17, 4, 5)
    assert cc.calibrate_cached(c, "abc123", ["batch"], root=str(tmp_path)) is False
    # recalibrate forces the measurement pass and rewrites the file
    d = _StubPlan(16, 4, 77)
    assert cc.calibrate_cached(d, "abc123", ["batch"], root=str(tmp_path), recalibrate=True) is False
    assert np.array_equal(cc.load(str(tmp_path / "abc123_Se16.json")).s_x, d.measured[:, 0])


def test_hit_with_wrong_layer_count_fails_loudly(tmp_path):
    cc.calibrate_cached(_StubPlan(8, 4, 1), "h", ["b"], root=str(tmp_path))
    with pytest.raises(ValueError):
        cc.calibrate_cached(_StubPlan(8, 5, 1), "h", ["b"], root=str(tmp_path))
