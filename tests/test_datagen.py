"""Seeded input generators: shapes, determinism, documented structure."""
import numpy as np

import oracle
from realtime_transformer_amd import datagen
from realtime_transformer_amd.configs import CONFIGS, FFNConfig


def test_bf16_bits_are_truncated_fp32_any_shape():
    rng = np.random.default_rng(0)
    for shape in [(7,), (3, 5), (2, 3, 4), (1, 256)]:
        x = rng.standard_normal(shape).astype(np.float32)
        b = datagen.to_bf16_bits(x)
        assert b.shape == x.shape and b.dtype == np.uint16
        assert np.array_equal(b, (x.view(np.uint32) >> 16).astype(np.uint16))
        back = oracle.bf16_to_f32(b)
        assert np.all(np.abs(back) <= np.abs(x)) and np.all(np.abs(x - back) <= np.abs(x) * 2.0 ** -7)


def test_deterministic_and_thread_independent():
    a = datagen.normal_f32(5, (1 << 22) + 1000)
    b = datagen.normal_f32(5, (1 << 22) + 1000)
    assert np.array_equal(a, b)
    # chunk c depends only on (seed, c)
    c = datagen.normal_f32(5, 1000)
    assert np.array_equal(a[:1000], c)


def test_single_block_inputs():
    cfg = CONFIGS[1]
    r, y = datagen.eval_inputs(cfg)
    assert r.shape == (16, 256) and y.shape == (16, 256)
    cal = datagen.calib_batches(cfg)
    assert len(cal) == 4 and all(c[0].shape == (16, 256) for c in cal)
    assert not np.array_equal(cal[0][0], r)
    rf = oracle.bf16_to_f32(r).astype(np.float64)
    assert abs(rf.std() - 1.0) < 0.1 and abs(rf.mean()) < 0.1


def test_chain_inputs_have_zero_prev_output():
    cfg = FFNConfig(2, "t", 50, 256, 512, 3, 0)
    r, y = datagen.eval_inputs(cfg)
    assert y is None and r.shape == (50, 256)


def test_text_rows_have_half_std():
    cfg = FFNConfig(3, "t", 788, 256, 512, 2, 0)
    r, _ = datagen.eval_inputs(cfg)
    rf = oracle.bf16_to_f32(r).astype(np.float64)
    assert abs(rf[:768].std() - 1.0) < 0.02
    assert abs(rf[768:].std() - 0.5) < 0.02


def test_outliers_exact_count_and_value():
    cfg = FFNConfig(5, "t", 64, 512, 512, 2, 2)
    r, _ = datagen.eval_inputs(cfg)
    rf = oracle.bf16_to_f32(r)
    k = (64 * 512) // 100
    assert int(np.sum(np.abs(rf) == 20.0)) == k
    assert 0.3 * k < int(np.sum(rf == 20.0)) < 0.7 * k


def test_weight_shapes_and_scale():
    cfg = FFNConfig(9, "t", 4, 256, 512, 2, 1)
    wg, wu, wd, wn = datagen.layer_weights(cfg, 1)
    assert wg.shape == (512, 256) and wu.shape == (512, 256) and wd.shape == (256, 512)
    assert wn.shape == (256,)
    assert abs(oracle.bf16_to_f32(wu).std() - 0.02) < 0.002
    assert abs(oracle.bf16_to_f32(wn).mean() - 1.0) < 0.02
    cfg2 = FFNConfig(9, "t", 4, 256, 512, 2, 2)
    assert datagen.layer_weights(cfg2, 1)[0] is None
