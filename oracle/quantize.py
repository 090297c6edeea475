"""Plain CPU oracle: rowwise fp8 (e4m3fn) quantisation of bf16 activations.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this module.  The GPU library shares no
code with it.

What is computed (the step just before the grouped GEMM, producing its XQ and
x_scale operands).  The pages fix the rowwise scheme (one scale per row of A,
constant along K: [MSLK-471], Design notes, scaling-scheme paragraph) but not how
the scales are chosen; the reading taken here is the usual amax one, stated with
the workloads: per row of x (bf16 values, widened exactly to fp32)

    s    = amax(|x|) / 448          in fp32, IEEE division; s = 1 if amax = 0
    y_k  = x_k / s                  in fp32, IEEE division
    q_k  = e4m3fn_rne(clamp(y_k, -448, 448))

448 is the largest finite e4m3fn value.  Every step that decides an integer code
is done in fp32, the precision of the GPU kernel, so the two agree bit for bit.
NaN inputs are outside the definition (amax ignores them; their codes are NaN).
"""
from __future__ import annotations

import numpy as np

from .grouped_gemm import bf16_bits_to_f64, e4m3fn_table

E4M3_MAX = np.float32(448.0)

# Positive finite e4m3fn values by code 0x00 .. 0x7E (increasing with the code).
_POS = e4m3fn_table()[:0x7F]


def e4m3fn_rne(y: np.ndarray) -> np.ndarray:
    """fp32 values with |y| <= 448 -> e4m3fn codes, round to nearest, ties to the
    even code (the even last mantissa bit; codes increase with the value, so the
    tie rule holds across binade boundaries too).  The sign bit is copied (-0
    gives 0x80)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    assert np.all(a[~np.isnan(a)] <= 448.0), "clamp before encoding"
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 0x7E)   # first code with value >= a
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = _POS[hi] - a
    d_lo = a - _POS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = np.where(np.isnan(a), np.uint8(0x7F), code)
    return (code | np.where(np.signbit(y), np.uint8(0x80), np.uint8(0))).astype(np.uint8)


def row_quotient(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """y[r, k] = x[r, k] / s[r]: one correctly rounded fp32 IEEE division per
    element (not a multiplication by a rounded reciprocal, which differs in the
    last bit for some inputs and so changes some codes)."""
    return (np.asarray(x, np.float32) / np.asarray(s, np.float32)[:, None]).astype(np.float32)


def quantize_rowwise(x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """x_bits: uint16 bf16 patterns [rows, K] -> (codes uint8 [rows, K], scales
    float32 [rows])."""
    x = bf16_bits_to_f64(np.asarray(x_bits, np.uint16)).astype(np.float32)
    rows = x.shape[0]
    if x.shape[1] == 0:
        return np.zeros(x.shape, np.uint8), np.ones(rows, np.float32)
    amax = np.nanmax(np.abs(x), axis=1).astype(np.float32)
    s = (amax / E4M3_MAX).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    y = row_quotient(x, s)
    y = np.where(y > E4M3_MAX, E4M3_MAX, np.where(y < -E4M3_MAX, -E4M3_MAX, y)).astype(np.float32)
    return e4m3fn_rne(y), s
