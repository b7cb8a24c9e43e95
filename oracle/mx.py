"""Oracle MX (microscaling) fp8 encoder/decoder, fp64.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the GPU path never does.

The pages name the MXFP8 format for the expert GEMMs (Mixture-of-Kittens
tweet by @rohanpaul_ai on the khabar-ai page: custom MXFP8 expert kernels;
dzen.guru page, megakernel paragraph of "Три решения…": BF16 and MXFP8
supported) without fixing its bits.  The workload recipe fixes them: E4M3
elements, one E8M0 scale per 32 contiguous elements along the reduction
dimension, round-to-nearest-even.  The scale rule is the one of the public
OCP Microscaling Formats (MX) v1.0 specification:

    X = floor(log2(amax)) - 8        (8 = exponent of the largest E4M3 power of two)
    X clamped to [-127, 127];  all-zero block -> X = -127
    element code = RNE_E4M3(clamp(v / 2^X, -448, 448)),  ties to the even code
    scale byte   = X + 127  (E8M0: 2^(byte - 127))

E4M3 ("fn" variant): sign, 4 exponent bits (bias 7), 3 mantissa bits, no
infinities, S.1111.111 is NaN, largest finite 448, smallest subnormal 2^-9.
The table below is built from that definition and nothing else.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code from the format definition (NaN for S.1111.111)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# Non-negative finite codes 0..126 in increasing value (the encoding is monotonic).
POS_VALUES = np.array([e4m3_value(c) for c in range(127)], dtype=np.float64)
# Full decode table for all 256 codes (NaN at 0x7F and 0xFF).
DECODE_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def encode_e4m3(s: np.ndarray) -> np.ndarray:
    """Saturating round-to-nearest-even of already-scaled fp64 values to E4M3 codes."""
    s = np.asarray(s, dtype=np.float64)
    a = np.minimum(np.abs(s), E4M3_MAX)
    hi = np.searchsorted(POS_VALUES, a, side="left")          # first table value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - POS_VALUES[lo]
    d_hi = POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    # the sign is kept, also when the magnitude rounds to zero (-0 -> 0x80)
    return (code | (np.signbit(s).astype(np.uint8) << 7)).astype(np.uint8)


def block_exponent(amax: np.ndarray) -> np.ndarray:
    """X = floor(log2 amax) - 8 from the fp64 exponent (frexp), clamped; -127 for zero blocks."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)                 # amax = m * 2^e with m in [0.5, 1)
    X = e.astype(np.int64) - 1 - 8
    X = np.where(amax > 0, X, -127)
    return np.clip(X, -127, 127)


def quantize(v: np.ndarray, axis: int = -1):
    """MX-quantise fp64 values along ``axis`` (length a multiple of 32).

    Returns (codes uint8 with v's shape, scales uint8 with that axis divided by 32)."""
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    K = v.shape[-1]
    if K % BLOCK:
        raise ValueError("MX length must be a multiple of 32")
    blk = v.reshape(v.shape[:-1] + (K // BLOCK, BLOCK))
    X = block_exponent(np.max(np.abs(blk), axis=-1))
    scaled = np.ldexp(blk, -X[..., None])          # exact power-of-two scaling
    codes = encode_e4m3(scaled).reshape(v.shape)
    scales = (X + 127).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(scales, -1, axis)


def dequantize(codes: np.ndarray, scales: np.ndarray, axis: int = -1) -> np.ndarray:
    """fp64 values of MX codes with their per-32 E8M0 scales along ``axis``."""
    c = np.moveaxis(np.asarray(codes, dtype=np.uint8), axis, -1)
    s = np.moveaxis(np.asarray(scales, dtype=np.uint8), axis, -1)
    K = c.shape[-1]
    vals = DECODE_TABLE[c].reshape(c.shape[:-1] + (K // BLOCK, BLOCK))
    out = np.ldexp(vals, s.astype(np.int64)[..., None] - 127).reshape(c.shape)
    return np.moveaxis(out, -1, axis)


def fake_quant(v: np.ndarray, axis: int = -1) -> np.ndarray:
    """dequantize(quantize(v)) along ``axis``."""
    c, s = quantize(v, axis)
    return dequantize(c, s, axis)
