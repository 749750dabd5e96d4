"""CPU oracle of INT8 per-row symmetric quantization and the INT8
matrix-vector product built on it.

TEST INFRASTRUCTURE. Only the tests and the benchmark's CPU-baseline leg may
import this module; the product path never calls it, and it shares no code
with the HIP kernels or their host library.

What it computes (page "RWKV-X Architecture", section "INT8 Quantization"):
every row of a linear projection's weight matrix W [out, in] gets its own
scale, the row's largest magnitude divided by 127, and each weight becomes
the integer nearest to weight / scale. At inference the input vector is
quantized once and every output row is an integer dot product, rescaled.

Readings where the section is silent (the same on the GPU side):

* arithmetic: the page's engine is single-precision C, so the scale and the
  quotient weight / scale are IEEE float32 operations (a quantized code is
  an integer decided by floating point, so both sides decide it in the same
  precision);
* "round" is C's roundf: to nearest, halves away from zero;
* an all-zero row has scale 0 and all codes 0 (the division is undefined);
* the input vector (one row per token of a batch) is quantized by the same
  rule as a weight row: its own scale max|x| / 127;
* an output element is (integer dot product) * w_scale[o] * x_scale[b]; here
  the dot product is exact (int64) and the rescaling float64.
"""
from __future__ import annotations

import numpy as np


def roundf(v: np.ndarray) -> np.ndarray:
    """C roundf on float32 values: nearest integer, halves away from zero.
    Written with floor and an exact fractional part: adding 0.5 first would
    round 0.49999997 up (0.49999997 + 0.5 is not representable)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)
    fl = np.floor(a)
    frac = a - fl                       # exact for |v| < 2**23
    r = fl + (frac >= np.float32(0.5)).astype(np.float32)
    return np.copysign(r, v).astype(np.float32)


def quantize_rows(x: np.ndarray):
    """Per-row symmetric INT8 quantization in float32.

    x: [rows, cols] (any float dtype; converted to float32 first, which is
    exact for bf16 and float32 inputs). Returns (q int8 [rows, cols],
    scale float32 [rows])."""
    x = np.asarray(x, dtype=np.float32)
    m = np.max(np.abs(x), axis=1)                       # exact
    scale = (m / np.float32(127.0)).astype(np.float32)  # IEEE float32 divide
    q = np.zeros(x.shape, dtype=np.int8)
    nz = scale > 0
    if np.any(nz):
        quot = (x[nz] / scale[nz, None]).astype(np.float32)
        q[nz] = roundf(quot).astype(np.int8)
    return q, scale


def q8_matmul(wq: np.ndarray, w_scale: np.ndarray, xq: np.ndarray,
              x_scale: np.ndarray) -> np.ndarray:
    """y[b, o] = (sum_i wq[o, i] * xq[b, i]) * w_scale[o] * x_scale[b].

    wq int8 [out, in], xq int8 [B, in]; the dot products are exact int64,
    the rescaling float64. Returns float64 [B, out]."""
    acc = xq.astype(np.int64) @ wq.astype(np.int64).T      # exact
    return acc.astype(np.float64) * w_scale.astype(np.float64)[None, :] \
        * x_scale.astype(np.float64)[:, None]


def q8_linear(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """The whole quantized projection: quantize W's rows and x's rows, then
    q8_matmul. Returns float64 [B, out]."""
    wq, ws = quantize_rows(w)
    xq, xs = quantize_rows(x)
    return q8_matmul(wq, ws, xq, xs)
