"""The five synthetic FFN-chain workloads (shapes, activation, layer count).

Each stands in for a workload the FlashRT pages run; none of the pages'
checkpoints or datasets is used:
  1 ffn_block_m16        single block, M=16, H=256, I=1024, GeGLU (tanh GELU)
  2 action_expert_m50    Pi0.5-style action expert: 18 layers, M=50, H=1024, I=4096, GeGLU
                         (itsolotime article, section 5.2: 18-layer gate/up fusion)
  3 vlm_prefix_m788      VLM prefix of 3 x 256 image tokens + 20 text tokens: 18 layers,
                         H=2048, I=16384, GeGLU (article section 6.2: 256 tokens per view;
                         section 7.2: 18 encoder FFN layers)
  4 llm_decode_m1        dense-LLM decode step: 64 layers, M=1, H=5120, I=17408, SwiGLU
                         (article section 8.1: 48 + 16 layer hybrid LLM, SwiGLU)
  5 dit_video_m4096      DiT video MLP: 30 layers, M=4096, H=3072, I=14336, GELU-tanh,
                         non-gated (project page table: video generation)
"""
from __future__ import annotations

from dataclasses import dataclass

ACT_GEGLU_TANH = 0
ACT_SWIGLU = 1
ACT_GELU_TANH = 2

ACT_NAMES = {ACT_GEGLU_TANH: "geglu_tanh", ACT_SWIGLU: "swiglu", ACT_GELU_TANH: "gelu_tanh"}


@dataclass(frozen=True)
class FFNConfig:
    index: int
    name: str
    M: int
    H: int
    I: int
    L: int
    act: int
    eps: float = 1e-6

    @property
    def gated(self) -> bool:
        return self.act != ACT_GELU_TANH

    # algorithmic work per layer: weights once, activations once per kernel,
    # unpadded M (K1: read R, Y, w_norm, write R, XQ; gate/up: read W, XQ,
    # write HQ; down: read W, HQ, write Y)
    def k1_bytes(self) -> int:
        return 7 * self.M * self.H + 2 * self.H

    def gateup_bytes(self) -> int:
        nw = 2 if self.gated else 1
        return nw * self.I * self.H + self.M * self.H + self.M * self.I

    def down_bytes(self) -> int:
        return self.I * self.H + self.M * self.I + 2 * self.M * self.H

    def layer_bytes(self) -> int:
        return self.k1_bytes() + self.gateup_bytes() + self.down_bytes()

    def gateup_flops(self) -> int:
        return (4 if self.gated else 2) * self.M * self.H * self.I

    def down_flops(self) -> int:
        return 2 * self.M * self.H * self.I

    def layer_flops(self) -> int:
        return self.gateup_flops() + self.down_flops()


CONFIGS = {
    1: FFNConfig(1, "ffn_block_m16", 16, 256, 1024, 1, ACT_GEGLU_TANH),
    2: FFNConfig(2, "action_expert_m50", 50, 1024, 4096, 18, ACT_GEGLU_TANH),
    3: FFNConfig(3, "vlm_prefix_m788", 788, 2048, 16384, 18, ACT_GEGLU_TANH),
    4: FFNConfig(4, "llm_decode_m1", 1, 5120, 17408, 64, ACT_SWIGLU),
    5: FFNConfig(5, "dit_video_m4096", 4096, 3072, 14336, 30, ACT_GELU_TANH),
}

BY_NAME = {c.name: c for c in CONFIGS.values()}


# ---------------------------------------------------------------------------
# Attention-input workloads (K1 + fused QKV projection + split + rotary
# embedding), one layer each.  Head layouts: the Pi0 / Pi0.5 specs' FusedQKV
# item interleaves 8 query heads and 1 key head (itsolotime article, section
# 5.2), read here as 8 query heads and 1 key/value head of dimension 256 for
# the action expert and the VLM prefix; the decode shape takes a grouped
# layout of 64 query and 8 key/value heads of dimension 128 at the decode
# chain's hidden size.  The residual inputs are those of the FFN workload of
# the same model (same seed index).
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class QkvConfig:
    index: int
    name: str
    M: int
    H: int
    nq: int
    nkv: int
    hd: int
    pos0: int          # rotary position of row 0 (row m takes pos0 + m)
    max_pos: int       # rotary table rows
    rope_base: float
    eps: float = 1e-6
    L: int = 1         # one layer (the generator then also draws a nonzero Y)

    @property
    def N(self) -> int:
        return (self.nq + 2 * self.nkv) * self.hd

    def k1_bytes(self) -> int:
        return 7 * self.M * self.H + 2 * self.H

    def qkv_bytes(self) -> int:
        # weights once, XQ, the positions, the table rows used, bf16 Q/K/V
        return self.N * self.H + self.M * self.H + 4 * self.M + self.M * self.hd * 4 + 2 * self.M * self.N

    def qkv_flops(self) -> int:
        return 2 * self.M * self.N * self.H


QKV_CONFIGS = {
    "qkv_action_expert_m50": QkvConfig(2, "qkv_action_expert_m50", 50, 1024, 8, 1, 256, 788, 1024, 10000.0),
    "qkv_vlm_prefix_m788": QkvConfig(3, "qkv_vlm_prefix_m788", 788, 2048, 8, 1, 256, 0, 1024, 10000.0),
    "qkv_llm_decode_m1": QkvConfig(4, "qkv_llm_decode_m1", 1, 5120, 64, 8, 128, 4095, 4096, 1e6),
}
