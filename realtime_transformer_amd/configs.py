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
