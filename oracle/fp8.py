"""Oracle for weight-only FP8 decode.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg; the product path never calls it.

Generation is bound by memory bandwidth, and storing the weights the decode steps
read as 8-bit floats halves their bytes (Chapter 11 "System Architecture &
Infrastructure at Scale", section "The Generation Bottleneck: Quantitative Analysis",
Table 11.4 and the optimisation list after it: INT8/FP8 weights for generation, with
little quality loss when sampling).  The pages fix no format; the reading taken here:

* format: OCP FP8 E4M3 ("e4m3fn": 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits, no infinities, largest finite value 448, subnormals down to 2^-9);
* weight-only, per output channel: for row n of a projection weight W [N, K] (the
  bf16 weight the decode step would use, LoRA folded), amax_n = max_k |W[n, k]|,
  scale_n = amax_n / 448 rounded to float32 (1 for an all-zero row), and
  q[n, k] = E4M3(W[n, k] / scale_n) with the quotient rounded to float32 and then to
  E4M3 by round-to-nearest-even, saturating at +-448;
* the decode projections (q/k/v, out, fc1, fc2) use W'[n, k] = q[n, k] * scale_n; the
  prompt pass, the LM head (the tied embedding) and everything else keep bf16.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_EXP = -6          # smallest normal exponent (2^-6); subnormal spacing 2^-9
E4M3_MANT = 3


def e4m3_round(y) -> np.ndarray:
    """Round float values to the nearest E4M3 value (ties to even), saturating at
    +-448; returns float64 holding the E4M3 values exactly."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    # spacing of the E4M3 grid around |y|: 2^(e - 3) for |y| in [2^e, 2^(e+1)), e >= -6;
    # 2^-9 below 2^-6 (subnormals).  frexp gives e exactly: |y| = f 2^(e+1), f in [1/2, 1)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex.astype(np.float64) - 1, E4M3_MIN_EXP)
    step = np.exp2(e - E4M3_MANT)
    m = a / step                                   # exact: step is a power of two
    r = np.floor(m)
    frac = m - r
    r = np.where((frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2) == 1)), r + 1, r)
    out = np.minimum(r * step, E4M3_MAX)
    return np.copysign(out, y)


def quantize_rows(W) -> Tuple[np.ndarray, np.ndarray]:
    """Per-output-channel E4M3 quantisation of W [N, K] (bf16 values given as any
    float type).  Returns (q [N, K] float64 E4M3 values, scale [N] float32)."""
    w32 = np.asarray(W, dtype=np.float32)
    amax = np.abs(w32).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (w32 / scale[:, None]).astype(np.float32)  # float32 quotient, correctly rounded
    return e4m3_round(y), scale


def dequantize(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """W' = q * scale in float64 (exact products)."""
    return np.asarray(q, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[:, None]


def fp8_weight(W) -> np.ndarray:
    """The decode step's weight under weight-only FP8: dequantize(quantize_rows(W))."""
    q, s = quantize_rows(W)
    return dequantize(q, s)
