"""FFNPlan: a plan over a torch-allocated workspace (memory and streams only).

PyTorch provides the device memory (one uint8 workspace tensor, staging
tensors for uploads) and the stream; every step of the FFN chain runs in
libfrt.  Slot accessors return torch views into the workspace at the fixed
addresses frt_ffn_io_get reports, so reading or writing a slot is a plain
device copy.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import _abi


def _require_gpu():
    if not torch.cuda.is_available():
        raise _abi.FrtError(_abi.FRT_ERR_UNSUPPORTED, "no HIP device visible")


def _to_dev_u16(a: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(device, non_blocking=False)


class FFNPlan:
    def __init__(self, M: int, H: int, I: int, L: int, act: int, eps: float = 1e-6,
                 device: int = 0, stream: Optional[torch.cuda.Stream] = None, flags: int = 0):
        _require_gpu()
        _abi.load()
        self.M, self.H, self.I, self.L, self.act = M, H, I, L, act
        self.gated = act != _abi.FRT_ACT_GELU_TANH
        # MXFP4 plans above 64 rows run the prefill GEMMs, whose activation
        # exponents sit in their own layout (rows padded to 128)
        self.mx_mm = bool(flags & _abi.FRT_FLAG_MXFP4) and M > 64
        self.device = torch.device("cuda", device)
        self.desc = _abi.make_desc(M, H, I, L, act, eps, device, flags)
        self.nbytes = _abi.frt_ffn_workspace_size(self.desc)
        self.ws = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=self.device)
        base = self.ws.data_ptr()
        self._off0 = (-base) % 256
        self.ws_ptr = base + self._off0
        self.plan = _abi.frt_ffn_plan_create(self.desc, self.ws_ptr, self.nbytes)
        self.io = _abi.frt_ffn_io_get(self.plan)
        self.stream = stream if stream is not None else torch.cuda.Stream(self.device)

    # ---- lifetime ---------------------------------------------------------
    def close(self):
        if getattr(self, "plan", None):
            torch.cuda.synchronize(self.device)
            _abi.frt_ffn_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def s(self) -> int:
        return self.stream.cuda_stream

    def sync(self):
        self.stream.synchronize()

    # ---- workspace views --------------------------------------------------
    def _view(self, ptr: int, nbytes: int) -> torch.Tensor:
        off = ptr - self.ws.data_ptr()
        assert 0 <= off and off + nbytes <= self.ws.numel()
        return self.ws[off:off + nbytes]

    def r_slot(self, l: int) -> torch.Tensor:
        n = self.M * self.H * 2
        return self._view(self.io.r_slots + l * self.io.stride_rh, n).view(torch.int16).view(self.M, self.H)

    def y_slot(self, l: int) -> torch.Tensor:
        n = self.M * self.H * 2
        return self._view(self.io.y_slots + l * self.io.stride_rh, n).view(torch.int16).view(self.M, self.H)

    def xq_slot(self, l: int) -> torch.Tensor:
        return self._view(self.io.xq_slots + l * self.io.stride_xq, self.M * self.H).view(self.M, self.H)

    def hq_slot(self, l: int) -> torch.Tensor:
        return self._view(self.io.hq_slots + l * self.io.stride_hq, self.M * self.I).view(self.M, self.I)

    def mod_slot(self, l: int) -> torch.Tensor:
        """Layer l's AdaRMSNorm modulation [2][H] (scale, shift) as int16 bf16 bits."""
        if not self.io.mod_slots:
            raise RuntimeError("plan has no modulation slots (FRT_FLAG_ADA_NORM not set)")
        return self._view(self.io.mod_slots + l * self.io.stride_mod, 2 * self.H * 2).view(torch.int16).view(2, self.H)

    def set_modulation(self, l: int, scale: np.ndarray, shift: np.ndarray):
        """Write layer l's scale and shift (numpy uint16 bf16 bits [H])."""
        v = np.stack([np.asarray(scale, np.uint16), np.asarray(shift, np.uint16)])
        with torch.cuda.stream(self.stream):
            self.mod_slot(l).copy_(_to_dev_u16(v, self.device))
        self.sync()

    def z(self) -> torch.Tensor:
        return self._view(self.io.z_out, self.M * self.H * 2).view(torch.int16).view(self.M, self.H)

    # ---- setup --------------------------------------------------------------
    def load_layer(self, layer: int, w_gate, w_up, w_down, w_norm):
        """Upload one layer's bf16 weights (numpy uint16 bit patterns) and quantise them."""
        tg = _to_dev_u16(w_gate, self.device) if w_gate is not None else None
        tu = _to_dev_u16(w_up, self.device)
        td = _to_dev_u16(w_down, self.device)
        tn = _to_dev_u16(w_norm, self.device)
        torch.cuda.synchronize(self.device)
        _abi.frt_quant_weights(self.plan, layer, tg.data_ptr() if tg is not None else None,
                               tu.data_ptr(), td.data_ptr(), tn.data_ptr(), self.s)
        del tg, tu, td, tn

    def set_awq(self, layer: int, s: np.ndarray):
        """MXFP4 plans: the layer's AWQ pre-scale (bf16 bits [H]); quantise the layer after it."""
        t = _to_dev_u16(s, self.device)
        torch.cuda.synchronize(self.device)
        _abi.frt_set_awq(self.plan, layer, t.data_ptr(), self.s)
        del t

    def export_mx(self, layer: int, which: int):
        """MXFP4 plans: (codes [rows][cols/2], exponents [rows][cols/32]) of gate (0), up (1), down (2)."""
        rows, cols = (self.H, self.I) if which == 2 else (self.I, self.H)
        return _abi.frt_export_mxfp4_weights(self.plan, layer, which, rows, cols)

    def _mx_slot(self, addr: int, K: int):
        # exponents in the kernels' layouts, gathered here into row-major
        # order (a copy).  GEMV (M <= 64, rows padded to 16): per (16-row
        # tile, four 128-K blocks) 64 lanes x 4 bytes, lane = 32-sub-block *
        # 16 + row % 16, byte = K block % 4.  Prefill (rows padded to 128):
        # per (64-row group, 128-K block) 64 lanes x 4 bytes, same lane,
        # byte = (row / 16) % 4.
        n = self.M * K // 2
        pad = 128 if self.mx_mm else 16
        mp = -(-self.M // pad) * pad
        v = self._view(addr, n + mp * K // 32)
        m = np.arange(self.M, dtype=np.int64)[:, None]
        b = np.arange(K // 32, dtype=np.int64)[None, :]
        if self.mx_mm:
            off = ((m >> 6) * (K // 128) + (b >> 2)) * 256 + ((b & 3) * 16 + (m & 15)) * 4 + ((m >> 4) & 3)
        else:
            off = (((m >> 4) * (K // 512) + (b >> 4)) * 64 + (b & 3) * 16 + (m & 15)) * 4 + ((b >> 2) & 3)
        idx = torch.as_tensor(off.reshape(-1), device=self.device)
        return v[:n].view(self.M, K // 2), v[n:][idx].view(self.M, K // 32)

    def xq_mx(self, l: int):
        """MXFP4 plans: XQ slot l as (codes [M][H/2] view, exponents [M][H/32]
        row-major copy) uint8."""
        return self._mx_slot(self.io.xq_slots + l * self.io.stride_xq, self.H)

    def hq_mx(self, l: int):
        """MXFP4 plans: HQ slot l as (codes [M][I/2], exponents [M][I/32]), as xq_mx."""
        return self._mx_slot(self.io.hq_slots + l * self.io.stride_hq, self.I)

    def path(self) -> int:
        """FRT_PATH_* bits of the kernels this plan's forward runs."""
        return _abi.frt_ffn_plan_path(self.plan)

    def export_codes(self, layer: int, which: int) -> np.ndarray:
        rows, cols = (self.H, self.I) if which == 2 else (self.I, self.H)
        return _abi.frt_export_weight_codes(self.plan, layer, which, rows, cols)

    def scales(self) -> np.ndarray:
        return _abi.frt_get_scales(self.plan, self.L)

    def set_act_scales(self, s_x: Sequence[float], s_h: Sequence[float]):
        a = np.stack([np.asarray(s_x, np.float32), np.asarray(s_h, np.float32)], axis=1)
        _abi.frt_set_act_scales(self.plan, a)

    def calibrate(self, batches, rows: Optional[int] = None, layer_begin: int = 0,
                  layer_end: Optional[int] = None):
        """batches: list of (r, y-or-None) numpy uint16 arrays [rows][H] entering layer_begin."""
        layer_end = self.L if layer_end is None else layer_end
        rows = rows if rows is not None else batches[0][0].shape[0]
        rs = [_to_dev_u16(r, self.device) for r, _ in batches]
        ys = None
        if batches[0][1] is not None:
            ys = [_to_dev_u16(y, self.device) for _, y in batches]
        torch.cuda.synchronize(self.device)
        _abi.frt_calibrate(self.plan, [t.data_ptr() for t in rs],
                           None if ys is None else [t.data_ptr() for t in ys], rows, layer_begin,
                           layer_end, self.s)
        del rs, ys

    def set_inputs(self, r0: np.ndarray, y0: Optional[np.ndarray]):
        with torch.cuda.stream(self.stream):
            self.r_slot(0).copy_(_to_dev_u16(r0, self.device))
            if y0 is None:
                self.y_slot(0).zero_()
            else:
                self.y_slot(0).copy_(_to_dev_u16(y0, self.device))
        self.sync()

    # ---- run ----------------------------------------------------------------
    def forward(self):
        _abi.frt_ffn_forward(self.plan, self.s)

    def forward_range(self, lb: int, le: int):
        _abi.frt_ffn_forward_range(self.plan, lb, le, self.s)

    def forward_profiled(self) -> np.ndarray:
        """Per-kernel milliseconds [L][3] (norm+quantise, gate/up, down) of one eager forward."""
        return _abi.frt_ffn_forward_profiled(self.plan, self.s, self.L)

    def time_kernel(self, which: int, reps: int = 3) -> float:
        """Average microseconds of kernel kind `which` (0 norm, 1 gate/up, 2 down)."""
        return _abi.frt_ffn_time_kernel(self.plan, which, reps, self.s)

    def capture(self):
        _abi.frt_graph_capture(self.plan, self.s)

    def replay(self):
        _abi.frt_graph_replay(self.plan, self.s)


def to_np_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def to_np_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


class QkvPlan:
    """Attention-input plan (include/frt_qkv.h) over a torch workspace tensor."""

    def __init__(self, M: int, H: int, nq: int, nkv: int, hd: int, max_pos: int, eps: float = 1e-6,
                 rope_base: float = 10000.0, device: int = 0, stream: Optional[torch.cuda.Stream] = None,
                 flags: int = 0):
        _require_gpu()
        _abi.load()
        self.M, self.H, self.nq, self.nkv, self.hd, self.max_pos = M, H, nq, nkv, hd, max_pos
        self.N = (nq + 2 * nkv) * hd
        self.device = torch.device("cuda", device)
        self.desc = _abi.make_qkv_desc(M, H, nq, nkv, hd, max_pos, eps, rope_base, device, flags)
        self.nbytes = _abi.frt_qkv_workspace_size(self.desc)
        self.ws = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=self.device)
        base = self.ws.data_ptr()
        self.ws_ptr = base + (-base) % 256
        self.plan = _abi.frt_qkv_plan_create(self.desc, self.ws_ptr, self.nbytes)
        self.io = _abi.frt_qkv_io_get(self.plan)
        self.stream = stream if stream is not None else torch.cuda.Stream(self.device)

    def close(self):
        if getattr(self, "plan", None):
            torch.cuda.synchronize(self.device)
            _abi.frt_qkv_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def s(self) -> int:
        return self.stream.cuda_stream

    def sync(self):
        self.stream.synchronize()

    def _view(self, ptr: int, nbytes: int) -> torch.Tensor:
        off = ptr - self.ws.data_ptr()
        assert 0 <= off and off + nbytes <= self.ws.numel()
        return self.ws[off:off + nbytes]

    def _u16(self, ptr, *shape) -> torch.Tensor:
        n = int(np.prod(shape))
        return self._view(ptr, 2 * n).view(torch.int16).view(*shape)

    def r_in(self):
        return self._u16(self.io.r_in, self.M, self.H)

    def y_in(self):
        return self._u16(self.io.y_in, self.M, self.H)

    def r_out(self):
        return self._u16(self.io.r_out, self.M, self.H)

    def xq(self):
        return self._view(self.io.xq, self.M * self.H).view(self.M, self.H)

    def q(self):
        return self._u16(self.io.q, self.M, self.nq, self.hd)

    def k(self):
        return self._u16(self.io.k, self.M, self.nkv, self.hd)

    def v(self):
        return self._u16(self.io.v, self.M, self.nkv, self.hd)

    def rope(self):
        return self._view(self.io.rope, self.max_pos * self.hd * 4).view(torch.float32).view(
            self.max_pos, self.hd // 2, 2)

    def mod(self):
        if not self.io.mod:
            raise RuntimeError("plan has no modulation slot (FRT_FLAG_ADA_NORM not set)")
        return self._u16(self.io.mod, 2, self.H)

    def load(self, wq, wk, wv, w_norm):
        tq, tk, tv, tn = (_to_dev_u16(a, self.device) for a in (wq, wk, wv, w_norm))
        torch.cuda.synchronize(self.device)
        _abi.frt_qkv_quant_weights(self.plan, tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), tn.data_ptr(), self.s)
        del tq, tk, tv, tn

    def export_codes(self) -> np.ndarray:
        return _abi.frt_qkv_export_weight_codes(self.plan, self.N, self.H)

    def scales(self) -> np.ndarray:
        return _abi.frt_qkv_get_scales(self.plan)

    def set_act_scale(self, s_x: float):
        _abi.frt_qkv_set_act_scale(self.plan, s_x)

    def set_modulation(self, scale: np.ndarray, shift: np.ndarray):
        v = np.stack([np.asarray(scale, np.uint16), np.asarray(shift, np.uint16)])
        with torch.cuda.stream(self.stream):
            self.mod().copy_(_to_dev_u16(v, self.device))
        self.sync()

    def calibrate(self, batches, rows: Optional[int] = None):
        rows = rows if rows is not None else batches[0][0].shape[0]
        rs = [_to_dev_u16(r, self.device) for r, _ in batches]
        ys = None if batches[0][1] is None else [_to_dev_u16(y, self.device) for _, y in batches]
        torch.cuda.synchronize(self.device)
        _abi.frt_qkv_calibrate(self.plan, [t.data_ptr() for t in rs], None if ys is None else [t.data_ptr() for t in ys],
                               rows, self.s)
        del rs, ys

    def set_inputs(self, r0: np.ndarray, y0: Optional[np.ndarray], pos: np.ndarray):
        with torch.cuda.stream(self.stream):
            self.r_in().copy_(_to_dev_u16(r0, self.device))
            if y0 is None:
                self.y_in().zero_()
            else:
                self.y_in().copy_(_to_dev_u16(y0, self.device))
        self.sync()
        _abi.frt_qkv_set_positions(self.plan, pos, self.s)

    def forward(self):
        _abi.frt_qkv_forward(self.plan, self.s)

    def time_kernel(self, which: int, reps: int = 10) -> float:
        return _abi.frt_qkv_time_kernel(self.plan, which, reps, self.s)

    def capture(self):
        _abi.frt_qkv_graph_capture(self.plan, self.s)

    def replay(self):
        _abi.frt_qkv_graph_replay(self.plan, self.s)

