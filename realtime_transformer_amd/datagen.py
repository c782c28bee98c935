"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This module only draws numbers and lays them out; it holds none of the FFN
block's arithmetic.  Draws use numpy's PCG64 through SeedSequence([seed,
chunk]) in fixed 4 Mi-element chunks (so the bytes do not depend on the thread
count).  A bf16 input is the top 16 bits of its fp32 draw (truncation toward
zero): a plain bit extraction, no rounding logic, which shifts each value by
less than 2^-8 of itself.

Distributions (one reading per workload):
  weights        W_gate, W_up [I,H], W_down [H,I] ~ N(0, 0.02) (std), bf16
  RMSNorm weight 1 + N(0, 0.1), bf16;  eps = 1e-6
  residual R[0]  N(0, 1) bf16; the M=788 prefix has rows 768..787 (20 text-like
                 tokens) at std 0.5; the M=4096 video chain has floor(1% of M*H)
                 distinct positions set to exactly +20 or -20 (fair coin)
  previous out   Y[0] ~ N(0,1) for the single block, zero for the chains
  calibration    4 batches drawn like the evaluation input, other seeds
  modulation     AdaRMSNorm scale and shift per layer [H] ~ N(0, 0.1), bf16
                 (stand-ins for a conditioning Dense layer's output)

Seeds: evaluation residual 1000*c, its Y[0] 1000*c + 50; calibration batch b
(1..4) 1000*c + b (and 1000*c + 50 + b for Y); layer l weights
1000*c + 100 + 4*l + {0 gate, 1 up, 2 down, 3 norm}; layer l modulation
2^20 + 1000*c + 2*l + {0 scale, 1 shift}.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Tuple

import numpy as np
from .configs import FFNConfig

_CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed: int, n: int) -> np.ndarray:
    """n standard normal fp32 draws, chunk c from PCG64(SeedSequence([seed, c]))."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(c):
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, c])))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 draws -> bf16 bit patterns (uint16): the top half of each fp32."""
    assert np.little_endian
    x = np.ascontiguousarray(x, dtype=np.float32)
    h = x.reshape(-1).view(np.uint16)
    return h[1::2].copy().reshape(x.shape)  # little-endian: odd halves are the high bits


def normal_bf16(seed: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    n = int(np.prod(shape))
    z = normal_f32(seed, n)
    if std != 1.0:
        z *= np.float32(std)
    if mean != 0.0:
        z += np.float32(mean)
    return to_bf16_bits(z).reshape(shape)


def residual(cfg: FFNConfig, seed: int) -> np.ndarray:
    """R[0] (or a calibration batch's residual): [M,H] bf16 bits."""
    M, H = cfg.M, cfg.H
    z = normal_f32(seed, M * H).reshape(M, H)
    if cfg.index == 3 and M > 768:
        # 3 x 256 image-like rows at std 1, then 20 text-like rows at std 0.5
        zt = normal_f32(seed + (1 << 24), (M - 768) * H).reshape(M - 768, H)
        z[768:] = zt * np.float32(0.5)
    if cfg.index == 5:
        k = (M * H) // 100
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1 << 30])))
        pos = g.choice(M * H, size=k, replace=False)
        sign = g.integers(0, 2, size=k)
        flat = z.reshape(-1)
        flat[pos] = np.where(sign == 1, np.float32(20.0), np.float32(-20.0))
    return to_bf16_bits(z)


def prev_output(cfg: FFNConfig, seed: int) -> Optional[np.ndarray]:
    """Y[0]: N(0,1) for the single-block workload, None (= zeros) for chains."""
    if cfg.L == 1:
        return normal_bf16(seed + 50, (cfg.M, cfg.H))
    return None


def eval_inputs(cfg: FFNConfig) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    s = 1000 * cfg.index
    return residual(cfg, s), prev_output(cfg, s)


def calib_batches(cfg: FFNConfig, nbatch: int = 4) -> List[Tuple[np.ndarray, Optional[np.ndarray]]]:
    out = []
    for b in range(1, nbatch + 1):
        s = 1000 * cfg.index + b
        out.append((residual(cfg, s), prev_output(cfg, s)))
    return out


def layer_seed(cfg: FFNConfig, layer: int, which: int) -> int:
    return 1000 * cfg.index + 100 + 4 * layer + which


def layer_weights(cfg: FFNConfig, layer: int):
    """(w_gate [I,H] or None, w_up [I,H], w_down [H,I], w_norm [H]) as bf16 bits."""
    H, I = cfg.H, cfg.I
    wg = normal_bf16(layer_seed(cfg, layer, 0), (I, H), std=0.02) if cfg.gated else None
    wu = normal_bf16(layer_seed(cfg, layer, 1), (I, H), std=0.02)
    wd = normal_bf16(layer_seed(cfg, layer, 2), (H, I), std=0.02)
    wn = normal_bf16(layer_seed(cfg, layer, 3), (H,), std=0.1, mean=1.0)
    return wg, wu, wd, wn


def modulation(cfg: FFNConfig, layer: int, std: float = 0.1) -> Tuple[np.ndarray, np.ndarray]:
    """(scale [H], shift [H]) bf16 bits for layer `layer`'s AdaRMSNorm."""
    base = (1 << 20) + 1000 * cfg.index + 2 * layer
    return normal_bf16(base, (cfg.H,), std=std), normal_bf16(base + 1, (cfg.H,), std=std)


def qkv_weights(cfg) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """(w_q [nq*hd, H], w_k [nkv*hd, H], w_v [nkv*hd, H], w_norm [H]) bf16 bits
    for an attention-input workload: projections N(0, 0.02), norm 1 + N(0, 0.1).
    Seeds 2^21 + 1000*c + {0 q, 1 k, 2 v, 3 norm}."""
    base = (1 << 21) + 1000 * cfg.index
    wq = normal_bf16(base, (cfg.nq * cfg.hd, cfg.H), std=0.02)
    wk = normal_bf16(base + 1, (cfg.nkv * cfg.hd, cfg.H), std=0.02)
    wv = normal_bf16(base + 2, (cfg.nkv * cfg.hd, cfg.H), std=0.02)
    wn = normal_bf16(base + 3, (cfg.H,), std=0.1, mean=1.0)
    return wq, wk, wv, wn


def positions(cfg) -> np.ndarray:
    """Rotary positions of the rows: pos0, pos0 + 1, ... (int32)."""
    return (cfg.pos0 + np.arange(cfg.M)).astype(np.int32)


def awq_scales(cfg, layer: int) -> np.ndarray:
    """AWQ pre-scale of layer `layer` for the MXFP4 variant: bf16 [H] of
    2^N(0, 0.5) per input channel (a stand-in for the per-channel activation
    statistics the pages' AWQ derives them from).  Seed 2^22 + 1000*c + l."""
    z = normal_f32((1 << 22) + 1000 * cfg.index + layer, cfg.H) * np.float32(0.5)
    return to_bf16_bits(np.exp2(z).astype(np.float32))
