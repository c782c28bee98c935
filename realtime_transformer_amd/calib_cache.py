"""On-disk cache of a plan's calibrated activation scales (JSON).

FlashRT's calibration framework (its homepage, "Calibration" under the
framework-layer description) keys a cache file by the checkpoint and the
sequence length, ``{ckpt_hash}_Se{N}.json``, in one directory shared by every
model; the file holds known fields plus a free-form ``extra`` map, and a hit
skips the measurement pass: the stored scales are baked straight into the
plan (the refit, alpha = activation scale x weight scale, is done by
``frt_set_act_scales``).  The same flow here:

  miss  plan.calibrate(batches) -> plan.scales() -> save()
  hit   load() -> plan.set_act_scales(s_x, s_h)

Key: ``ckpt_hash`` is a SHA-256 over the plan-independent description of the
weights (every layer's bf16 tensors with their shapes, in layer order) and
the settings that change what the scales measure (activation, eps, the
norm-variant flags); ``N`` is the plan's M.  With AdaRMSNorm the modulation
in the slots during calibration is part of the calibration sample, not of the
key.  Scales are float32 values written as JSON numbers (shortest repr of the
exactly widened double), so a load gives back the same bits.
"""
from __future__ import annotations

import hashlib
import json
import math
import os
import tempfile
from dataclasses import dataclass, field
from typing import Any, Dict, Iterable, Optional, Sequence

import numpy as np

FORMAT_VERSION = 1
ENV_DIR = "FRT_CALIB_DIR"
# flag bits that change the activation scales (the rest only pick kernels)
_SCALE_FLAGS = 8 | 16  # FRT_FLAG_NORM_FUSE | FRT_FLAG_ADA_NORM


def default_dir() -> str:
    d = os.environ.get(ENV_DIR)
    return d if d else os.path.join(os.path.expanduser("~"), ".realtime_transformer_amd", "calibration")


class CkptHasher:
    """Incremental checkpoint hash: feed each layer's tensors in order."""

    def __init__(self, H: int, I: int, L: int, act: int, eps: float, flags: int = 0):
        self._h = hashlib.sha256()
        hdr = {"H": int(H), "I": int(I), "L": int(L), "act": int(act),
               "eps": float(np.float32(eps)).hex(), "flags": int(flags) & _SCALE_FLAGS}
        self._h.update(json.dumps(hdr, sort_keys=True).encode())
        self._layers = 0

    def add_layer(self, tensors: Sequence[Optional[np.ndarray]]):
        self._h.update(b"L%d" % self._layers)
        for t in tensors:
            if t is None:
                self._h.update(b"N")
                continue
            a = np.ascontiguousarray(t)
            self._h.update(("%s%s" % (a.dtype.str, a.shape)).encode())
            self._h.update(a.view(np.uint8).reshape(-1).data)
        self._layers += 1

    def hexdigest(self, n: int = 16) -> str:
        return self._h.hexdigest()[:n]


def ckpt_hash(H: int, I: int, L: int, act: int, eps: float, layers: Iterable[Sequence[Optional[np.ndarray]]],
              flags: int = 0) -> str:
    h = CkptHasher(H, I, L, act, eps, flags)
    for t in layers:
        h.add_layer(t)
    return h.hexdigest()


def cache_path(ckpt: str, N: int, root: Optional[str] = None) -> str:
    if not ckpt or any(c in ckpt for c in "/\\."):
        raise ValueError("bad checkpoint hash %r" % (ckpt,))
    if int(N) < 1:
        raise ValueError("sequence length must be >= 1")
    return os.path.join(root or default_dir(), "%s_Se%d.json" % (ckpt, int(N)))


@dataclass
class CalibRecord:
    ckpt_hash: str
    seq: int
    s_x: np.ndarray          # float32 [L] activation scale entering each gate/up GEMM
    s_h: np.ndarray          # float32 [L] activation scale entering each down GEMM
    s_w: Optional[np.ndarray] = None   # float32 [L][3] weight scales (gate, up, down), informational
    extra: Dict[str, Any] = field(default_factory=dict)

    @property
    def L(self) -> int:
        return int(self.s_x.shape[0])


def _check_scales(name: str, v) -> np.ndarray:
    a = np.asarray(v, dtype=np.float64)
    if a.ndim != 1 or a.size == 0:
        raise ValueError("%s: expected a non-empty list" % name)
    if not np.all(np.isfinite(a)) or np.any(a <= 0):
        raise ValueError("%s: scales must be finite and > 0" % name)
    f = a.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), a):
        raise ValueError("%s: values are not float32" % name)
    return f


def save(path: str, rec: CalibRecord) -> str:
    """Write atomically (temporary file in the same directory, then rename)."""
    s_x = _check_scales("s_x", rec.s_x)
    s_h = _check_scales("s_h", rec.s_h)
    if s_x.shape != s_h.shape:
        raise ValueError("s_x and s_h differ in length")
    doc = {"format": FORMAT_VERSION, "ckpt_hash": rec.ckpt_hash, "seq": int(rec.seq), "layers": int(s_x.size),
           "s_x": [float(v) for v in s_x], "s_h": [float(v) for v in s_h],
           "s_w": None if rec.s_w is None else [[float(v) for v in row] for row in np.asarray(rec.s_w, np.float32)],
           "extra": dict(rec.extra)}
    text = json.dumps(doc, indent=1, allow_nan=False)
    d = os.path.dirname(os.path.abspath(path))
    os.makedirs(d, exist_ok=True)
    fd, tmp = tempfile.mkstemp(prefix=".calib-", suffix=".json", dir=d)
    try:
        with os.fdopen(fd, "w") as f:
            f.write(text)
        os.replace(tmp, path)
    except BaseException:
        if os.path.exists(tmp):
            os.unlink(tmp)
        raise
    return path


def load(path: str, expect_ckpt: Optional[str] = None, expect_seq: Optional[int] = None,
         expect_layers: Optional[int] = None) -> CalibRecord:
    """Parse and validate; raises ValueError on a malformed or mismatched file."""
    with open(path) as f:
        doc = json.load(f)
    if not isinstance(doc, dict) or doc.get("format") != FORMAT_VERSION:
        raise ValueError("%s: unknown calibration format" % path)
    s_x = _check_scales("s_x", doc.get("s_x"))
    s_h = _check_scales("s_h", doc.get("s_h"))
    if s_x.size != s_h.size or s_x.size != doc.get("layers"):
        raise ValueError("%s: layer count mismatch" % path)
    if expect_layers is not None and s_x.size != expect_layers:
        raise ValueError("%s: %d layers, plan has %d" % (path, s_x.size, expect_layers))
    if expect_ckpt is not None and doc.get("ckpt_hash") != expect_ckpt:
        raise ValueError("%s: checkpoint hash mismatch" % path)
    if expect_seq is not None and doc.get("seq") != int(expect_seq):
        raise ValueError("%s: sequence length mismatch" % path)
    s_w = doc.get("s_w")
    s_w = None if s_w is None else np.asarray(s_w, np.float32)
    extra = doc.get("extra") or {}
    if not isinstance(extra, dict):
        raise ValueError("%s: extra must be a map" % path)
    return CalibRecord(doc["ckpt_hash"], int(doc["seq"]), s_x, s_h, s_w, extra)


def calibrate_cached(plan, ckpt: str, batches, root: Optional[str] = None, recalibrate: bool = False,
                     extra: Optional[Dict[str, Any]] = None) -> bool:
    """Install activation scales on `plan` from the cache, or measure and
    store them.  Returns True on a cache hit.  `batches` are the calibration
    inputs for FFNPlan.calibrate (only read on a miss)."""
    path = cache_path(ckpt, plan.M, root)
    if not recalibrate and os.path.exists(path):
        rec = load(path, expect_ckpt=ckpt, expect_seq=plan.M, expect_layers=plan.L)
        plan.set_act_scales(rec.s_x, rec.s_h)
        return True
    plan.calibrate(batches)
    sc = plan.scales()
    rec = CalibRecord(ckpt, plan.M, sc[:, 0].copy(), sc[:, 3].copy(), sc[:, [1, 2, 4]].copy(), dict(extra or {}))
    save(path, rec)
    return False
