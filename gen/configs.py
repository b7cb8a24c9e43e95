"""Workload shapes for the single-GPU MoE layer.

Every workload is synthetic.  The shapes follow the pages' setting: one GPU's
share of a DeepSeek-V3-like MoE layer at 2,048 pre-routing tokens (Mixture-of-
Kittens benchmark paragraph, "Что показали замеры?" on the dzen.guru page), a
small-batch decode (the warp-decode page, toolnavs.com), a tiny fp32 case
small enough for a per-token brute force, and a skewed-load training case.

Symbols: T tokens, d hidden, E experts, k top-k, f expert intermediate size,
fs shared-expert intermediate size (0 = none), C ring capacity in rows.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d: int
    E: int
    k: int
    f: int
    dtype: str = "bf16"          # "f32" | "bf16" | "mxfp8"
    fs: int = 0                  # shared expert width (decode only)
    zipf_s: float = 0.0          # >0: router biases skew expert popularity
    hot_ratio: float = 0.0       # target hottest-expert load / mean load
    backward: bool = False       # also draw dY
    capacity_factor: float = 1.25
    margin: float = 1e-3         # redraw tokens whose k-th/(k+1)-th logit gap is below this
    cid: int = 0                 # seed-substream id of the workload

    @property
    def n(self) -> int:
        """Token copies after routing."""
        return self.T * self.k

    @property
    def C(self) -> int:
        """Ring capacity: 1.25x the mean expert load summed over experts, no per-expert cap."""
        return int(math.ceil(self.capacity_factor * self.n))

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


# The tiny fp32 forward: every tensor fp32, small enough for the per-token brute force.
TINY_F32 = LayerConfig("tiny_f32", T=16, d=128, E=8, k=2, f=256, dtype="f32", cid=0)

# Small-batch decode: bf16 weights, fp32 accumulate, one always-on shared expert.
def DECODE(B: int) -> LayerConfig:
    return LayerConfig(f"decode_b{B}", T=B, d=7168, E=256, k=8, f=2048, fs=2048,
                       dtype="bf16", cid=1)

# 2,048-token training-share forward (DeepSeek-V3-like expert shapes), bf16 and MXFP8.
FWD_BF16 = LayerConfig("fwd_bf16_t2048", T=2048, d=7168, E=256, k=8, f=2048,
                       dtype="bf16", cid=2)
FWD_MXFP8 = FWD_BF16.with_(name="fwd_mxfp8_t2048", dtype="mxfp8", cid=3)

# Skewed-load forward + backward: Zipf-shaped expert popularity, hottest ~8x mean.
SKEW_BWD = LayerConfig("skew_bwd_t8192", T=8192, d=4096, E=512, k=10, f=1024,
                       dtype="bf16", zipf_s=1.1, hot_ratio=8.0, backward=True, cid=4)


@dataclass(frozen=True)
class ShareConfig:
    """One GPU's expert-parallel share of the 2,048-token layer on 64 GPUs:
    4 local experts receiving 16,384 token copies in total (multinomial counts)."""
    name: str = "share_bf16_e4"
    rows: int = 16384
    d: int = 7168
    E: int = 4
    f: int = 2048
    dtype: str = "bf16"
    capacity_factor: float = 1.25
    cid: int = 5

    @property
    def C(self) -> int:
        return int(math.ceil(self.capacity_factor * self.rows))


SHARE_BF16 = ShareConfig()
SHARE_MXFP8 = ShareConfig(name="share_mxfp8_e4", dtype="mxfp8", cid=6)

ALL = {c.name: c for c in [TINY_F32, DECODE(1), DECODE(4), DECODE(8), FWD_BF16, FWD_MXFP8, SKEW_BWD]}
