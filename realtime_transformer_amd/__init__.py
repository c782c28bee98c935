"""realtime_transformer_amd: the fused FP8 transformer-FFN chain for AMD MI355X.

The hot path (residual add + RMSNorm + E4M3 quantise, FP8 gate/up GEMM with
the gated activation and re-quantisation fused, FP8 down GEMM, chained over
layers and replayed as one HIP graph) lives in libfrt.so behind the C ABI of
include/frt_ffn.h.  ``_abi`` is the ctypes binding with the same names;
``plan.FFNPlan`` owns a torch-allocated workspace; ``datagen`` draws the seeded
synthetic inputs; ``configs`` names the five workloads.
"""
from .configs import CONFIGS, BY_NAME, FFNConfig  # noqa: F401
from . import _abi  # noqa: F401
from ._abi import FrtError  # noqa: F401
