"""Plain CPU oracle: FP8 (e4m3fn) grouped GEMM with block (groupwise) scaling.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this module.  The GPU library shares no
code with it.

What is computed ([MSLK-471], first commit of the list, on the two scaling
schemes): block scaling carries one scale per (scale_block_k x scale_block_n)
block of B, so each block's partial sum is scaled inside the K loop rather than
once after it.  The pages leave A's scale granularity open; the reading taken here
is one scale per row of A and K block.  Stacked layout, per group g and row m of
g, with bk = scale_block_k, bn = scale_block_n:

    Y[m, n] = sum_kb ( sum_{k in block kb} dec(XQ[m, k]) dec(WQ[g, n, k]) )
                     * x_scale[m, kb] * w_scale[g, n // bn, kb]          -> bf16

x_scale is [total_M, K / bk], w_scale [G, N / bn, K / bk]; K and N must be whole
numbers of blocks (the pages require the block bound under block scaling).

Arithmetic: each block's partial sum is exact in fp64 (as for the rowwise
oracle); it is scaled in fp64, (acc_kb * x_scale) * w_scale, the scaled partials
are added in fp64 in ascending kb, and the sum is rounded to bf16 once (RNE).
Unlike the rowwise case the fp64 sum of scaled partials is not exact in general;
its error is about 2^-52 relative, far below a bf16 ulp.
"""
from __future__ import annotations

import numpy as np

from .grouped_gemm import (ROW_UNTOUCHED, ROW_WRITTEN, ROW_ZEROED, UNTOUCHED_SENTINEL, OracleResult,
                           _accumulate, bf16_rne_from_f64, offsets_row_groups, stacked_row_groups)


def column_blocks(N: int, block_n: int) -> np.ndarray:
    """Scale block of each output column: n // block_n."""
    return np.arange(N) // block_n


def block_partials(a_codes: np.ndarray, b_codes: np.ndarray, block_k: int) -> np.ndarray:
    """acc[kb, m, n] = sum over block kb of dec(a[m, k]) dec(b[n, k]), exact in fp64."""
    K = a_codes.shape[1]
    nkb = K // block_k
    return np.stack([_accumulate(a_codes[:, kb * block_k:(kb + 1) * block_k],
                                 b_codes[:, kb * block_k:(kb + 1) * block_k]) for kb in range(nkb)])


def scale_blocks(partials: np.ndarray, xs: np.ndarray, ws_cols: np.ndarray) -> np.ndarray:
    """sum_kb (partials[kb] * xs[:, kb]) * ws_cols[:, kb], in fp64, ascending kb.
    xs: [rows, nkb]; ws_cols: [n, nkb] (each column's block scale)."""
    xs = np.asarray(xs, np.float64)
    ws_cols = np.asarray(ws_cols, np.float64)
    out = np.zeros(partials.shape[1:])
    for kb in range(partials.shape[0]):
        out += (partials[kb] * xs[:, kb][:, None]) * ws_cols[:, kb][None, :]
    return out


def grouped_stacked_blockscale(XQ, WQ, x_scale, w_scale, M_sizes, block_k: int = 128,
                               block_n: int = 128) -> OracleResult:
    """Stacked layout with block scales: XQ [total_M, K], WQ [G, N, K], x_scale
    [total_M, K / block_k], w_scale [G, N / block_n, K / block_k], M_sizes [G]
    -> Y [total_M, N]; rows of no group untouched."""
    XQ = np.asarray(XQ, np.uint8)
    return _packed_blockscale(XQ, WQ, x_scale, w_scale, stacked_row_groups(M_sizes, XQ.shape[0]), block_k, block_n)


def grouped_offsets_blockscale(XQ, WQ, x_scale, w_scale, offsets, block_k: int = 128,
                               block_n: int = 128) -> OracleResult:
    """Offsets layout (int32 inclusive prefix of the group row counts) with block
    scales; otherwise as grouped_stacked_blockscale."""
    XQ = np.asarray(XQ, np.uint8)
    return _packed_blockscale(XQ, WQ, x_scale, w_scale, offsets_row_groups(offsets, XQ.shape[0]), block_k, block_n)


def grouped_batched_blockscale(XQ, WQ, x_scale, w_scale, block_k: int = 128, block_n: int = 128) -> OracleResult:
    """Batched layout with block scales: XQ [G, M, K], x_scale [G, M, K / block_k],
    every group a full slab of M rows -> Y [G, M, N] (flattened row classes)."""
    XQ = np.asarray(XQ, np.uint8)
    G, M, K = XQ.shape
    owner = np.repeat(np.arange(G, dtype=np.int64), M)
    res = _packed_blockscale(XQ.reshape(G * M, K), WQ, np.asarray(x_scale, np.float32).reshape(G * M, -1),
                             w_scale, owner, block_k, block_n)
    N = np.asarray(WQ).shape[1]
    return OracleResult(res.values.reshape(G, M, N), res.bits.reshape(G, M, N), res.row_class)


def _packed_blockscale(XQ, WQ, x_scale, w_scale, owner, block_k, block_n) -> OracleResult:
    """Groups packed along M with block scales; owner[r] is the group of row r (-1: none)."""
    WQ = np.asarray(WQ, np.uint8)
    total_M, K = XQ.shape
    G, N, K2 = WQ.shape
    assert K == K2 and K % block_k == 0 and N % block_n == 0
    x_scale = np.asarray(x_scale, np.float32)
    w_scale = np.asarray(w_scale, np.float32)
    assert x_scale.shape == (total_M, K // block_k) and w_scale.shape == (G, N // block_n, K // block_k)
    values = np.full((total_M, N), np.nan)
    bits = np.full((total_M, N), UNTOUCHED_SENTINEL, dtype=np.uint16)
    row_class = np.full(total_M, ROW_UNTOUCHED, dtype=np.int8)
    if K == 0:
        return OracleResult(np.zeros((total_M, N)), np.zeros((total_M, N), np.uint16),
                            np.full(total_M, ROW_ZEROED, np.int8))
    col_block = column_blocks(N, block_n)
    for g in range(G):
        rows = np.nonzero(owner == g)[0]
        if rows.size == 0:
            continue
        part = block_partials(XQ[rows], WQ[g], block_k)
        v = scale_blocks(part, x_scale[rows], w_scale[g][col_block])
        values[rows] = v
        bits[rows] = bf16_rne_from_f64(v)
        row_class[rows] = ROW_WRITTEN
    return OracleResult(values, bits, row_class)


def grouped_dynamic_blockscale(XQ, WQ, x_scale, w_scale, zero_start_index_M, zeroing_output_tensor: bool = True,
                               block_k: int = 128, block_n: int = 128) -> OracleResult:
    """Padded layout with block scales: XQ [G, em, K], WQ [G, N, K], x_scale
    [G, em, K / block_k], w_scale [G, N / block_n, K / block_k], zero_start_index_M
    [G] -> Y [G, em, N].  Row i of slab g is valid if i < clamp(zsi[g], 0, em);
    padding rows are zero when zeroing_output_tensor, else untouched (flattened
    row classes [G * em])."""
    XQ = np.asarray(XQ, np.uint8)
    WQ = np.asarray(WQ, np.uint8)
    G, em, K = XQ.shape
    G2, N, K2 = WQ.shape
    assert G == G2 and K == K2 and K % block_k == 0 and N % block_n == 0
    x_scale = np.asarray(x_scale, np.float32)
    w_scale = np.asarray(w_scale, np.float32)
    assert x_scale.shape == (G, em, K // block_k) and w_scale.shape == (G, N // block_n, K // block_k)
    if K == 0:
        return OracleResult(np.zeros((G, em, N)), np.zeros((G, em, N), np.uint16),
                            np.full(G * em, ROW_ZEROED, np.int8))
    valid = np.clip(np.asarray(zero_start_index_M, np.int64), 0, em)
    values = np.full((G, em, N), np.nan)
    bits = np.full((G, em, N), UNTOUCHED_SENTINEL, dtype=np.uint16)
    row_class = np.full((G, em), ROW_UNTOUCHED, np.int8)
    col_block = column_blocks(N, block_n)
    for g in range(G):
        v = int(valid[g])
        if v:
            part = block_partials(XQ[g, :v], WQ[g], block_k)
            out = scale_blocks(part, x_scale[g, :v], w_scale[g][col_block])
            values[g, :v] = out
            bits[g, :v] = bf16_rne_from_f64(out)
            row_class[g, :v] = ROW_WRITTEN
        if zeroing_output_tensor and v < em:
            values[g, v:] = 0.0
            bits[g, v:] = 0
            row_class[g, v:] = ROW_ZEROED
    return OracleResult(values, bits, row_class.reshape(-1))
