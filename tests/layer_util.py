"""Helpers shared by the GPU parity tests: hand the GPU's exact inputs to the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from gen import bits16


def to_oracle(t: torch.Tensor) -> np.ndarray:
    """fp64 host copy decoded by the oracle from the raw bits (bf16 or fp32)."""
    if t.dtype == torch.bfloat16:
        return oracle.from_bf16_bits(bits16(t))
    return oracle.from_f32(t.detach().float().cpu().numpy())


def mx_scale_rows(s: torch.Tensor) -> torch.Tensor:
    """The library's MX scale layout [cols/128][rows][4] as the row layout [rows, cols/32]
    the oracle uses (a pure relabelling of bytes)."""
    g, r, _ = s.shape
    return s.permute(1, 0, 2).reshape(r, g * 4)


class LazyWeights:
    """Oracle weight accessor e -> (W_gate[e], W_up[e], W_down[e]) in fp64, one expert at
    a time from device tensors (MX: decoded by the oracle's own table from codes/scales)."""

    def __init__(self, wg, wu, wd, mx_codes=None):
        self.wg, self.wu, self.wd = wg, wu, wd
        # ((cg, sg), (cu, su), (cd, sd)) device tensors or None; scales as [E, rows, cols/32]
        self.mx = None if mx_codes is None else tuple(
            (c, mx_scale_rows(sc).reshape(c.shape[0], c.shape[1], c.shape[2] // 32)) for c, sc in mx_codes)
        self.cache = {}

    def __call__(self, e):
        if e not in self.cache:
            if len(self.cache) > 4:
                self.cache.clear()
            if self.mx is None:
                self.cache[e] = tuple(to_oracle(w[e]) for w in (self.wg, self.wu, self.wd))
            else:
                self.cache[e] = tuple(
                    oracle.mx.dequantize(c[e].cpu().numpy(), s[e].cpu().numpy(), axis=1)
                    for c, s in self.mx)
        return self.cache[e]

    def oracle_mx(self, e):
        """The oracle's own MX quantisation of expert e's bf16 weights (codes, scales) x 3."""
        return tuple(oracle.mx.quantize(to_oracle(w[e]), axis=1) for w in (self.wg, self.wu, self.wd))


def rel(got, ref) -> float:
    return oracle.max_abs_rel(np.asarray(got, dtype=np.float64), ref)
