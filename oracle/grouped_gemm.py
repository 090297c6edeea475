"""Plain CPU oracle: FP8 (e4m3fn) x FP8 rowwise-scaled grouped GEMM -> bf16.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this module.  The GPU library shares no
code with it: no kernels, headers, tables or helpers.

Sources (web pages; cited by title and section):
  [MSLK-471]  "Back the FP8 rowwise grouped GEMM ops with FlyDSL on ROCm",
              meta-pytorch/MSLK pull request 471.
  [FlyDSL-913] "Port GEMM/MoE/conv kernels to the layout API",
              ROCm/FlyDSL pull request 913.

What is computed, per group g (the plain definition, written out):

    Y_g = (dec(XQ_g) @ dec(WQ_g)^T) * x_scale[m] * w_scale[g, n]     -> bf16

  * Rowwise scaling: one scale per row of A and one per output column (row of
    W), both constant along K, so they factor out of the reduction and are
    applied once after it ([MSLK-471], Design notes, scaling-scheme paragraph;
    and the first commit of the list, on the rowwise scheme).
  * Stacked layout: groups packed densely along M, group g owning the next
    M_sizes[g] rows ([MSLK-471], Summary op table, "_stacked" row: [G] int64 row
    counts; commit adding the layout enum, layout "sizes").
  * Padded ("dynamic") layout: each group owns a slab of expected_m rows of which
    only the first zero_start_index_M[g] are valid; padding rows are zero, the
    part of the contract the zeroing_output_tensor flag controls ([MSLK-471],
    commits adding the padded layout and its test).
  * Offsets layout (2D-3D): groups packed along M as in the stacked layout, but
    the boundaries come as an int32 inclusive prefix sum: group g owns rows
    [offsets[g-1], offsets[g]) with offsets[-1] = 0 ([MSLK-471], commit adding
    the offsets layout, and the commit mapping the grouped mm op's 2D-3D ranks
    onto it).
  * Batched layout (3D-3D): every group owns a full slab of M rows, all valid;
    there is no row metadata ([MSLK-471], commit adding the batched layout).
  * N-offsets layout (3D-2D): the weights are one [total_N, K] matrix whose rows
    (output columns) the groups partition by an int32 inclusive prefix; group g
    multiplies its own slab XQ[g] [M, K] against its rows of W, and the results
    sit side by side in Y [M, total_N] ([MSLK-471], commit adding the 3D-2D form
    of the grouped mm; commit on store predicates keyed on the last column).
  * K-offsets layout (2D-2D): both operands are one matrix, XQ [M, total_K] and
    WQ [N, total_K], whose K columns the groups slice by an int32 inclusive
    prefix; every group contracts over its own slice only and produces a whole
    [M, N] output, so Y is [G, M, N] ([MSLK-471], commit adding the 2D-2D form,
    and the commit keying the K-tail predicate on the group's own slice).
  * A contraction over K = 0 returns a zeroed output whatever the layout
    ([MSLK-471], commits on zero-length reductions and on the fakes' contracts).

Arithmetic (precision chosen so the oracle is exact up to its final rounding):
  1. e4m3fn codes are decoded through a 256-entry fp64 table built from the bit
     definition (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0
     is subnormal; 0x7F and 0xFF are NaN; no infinities).
  2. For each group, one fp64 matmul of the decoded, UNSCALED operands.  Every
     product is a multiple of 2^-18 below 2^18, so for K < 171196 every partial
     sum fits in 53 bits and the fp64 result is exact in any summation order
     (BLAS allowed).
  3. Scales are applied in fp64: (acc * x_scale[m]) * w_scale[g, n].
  4. Rounded to bf16 directly from fp64 with round-to-nearest-even (no detour
     through fp32, which could round twice).

Readings taken where the pages are silent (also listed in the design notes):
  * M_sizes entries < 0 count as 0; rows past the running sum (or past total_M)
    belong to no group and are left untouched.
  * zero_start_index_M is clamped to [0, expected_m].
  * offsets: group g ends at min(max(offsets[g], end of group g-1), total_M), so
    an offset below its predecessor makes an empty group and rows past the last
    end belong to no group (left untouched).
  * K = 0 zeroes every row of the output, in every layout.
  * n_offsets, k_offsets: the boundaries are read like the offsets layout's (an
    end below its predecessor makes an empty group, ends are cut at total_N or
    total_K); columns past the last end belong to no group and are untouched.
    An empty K slice contributes a zero sum, scaled as usual.
  * Scales of the two new layouts: n_offsets takes x_scale [G, M] (one per row of
    each slab) and w_scale [total_N] (one per row of W); k_offsets takes x_scale
    [G, M] and w_scale [G, N], since each group's slice of a row is a separate
    quantised vector (the pages name no scale shapes for these ranks).

Row classes returned with every result: ROW_WRITTEN (computed), ROW_ZEROED
(must be +-0), ROW_UNTOUCHED (the caller's buffer is left as it was).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ROW_UNTOUCHED = 0
ROW_WRITTEN = 1
ROW_ZEROED = 2

_E4M3_BIAS = 7


# ---------------------------------------------------------------------------
# 1. e4m3fn decode (OCP 8-bit floating point, E4M3 "fn" variant: finite + NaN).
# ---------------------------------------------------------------------------

def _build_e4m3fn_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if (code >> 7) & 1 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            t[code] = np.nan
        elif exp == 0:
            t[code] = sign * man * 2.0 ** (1 - _E4M3_BIAS - 3)   # subnormal: m * 2^-9
        else:
            t[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - _E4M3_BIAS)
    return t


_E4M3FN_TABLE = _build_e4m3fn_table()


def e4m3fn_table() -> np.ndarray:
    """Copy of the 256-entry fp64 decode table (index = byte code)."""
    return _E4M3FN_TABLE.copy()


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """uint8 e4m3fn codes -> fp64 values (exact)."""
    return _E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


# ---------------------------------------------------------------------------
# 4. fp64 -> bf16, round to nearest, ties to even, in one step.
# ---------------------------------------------------------------------------

def bf16_rne_from_f64(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (RNE) and return the uint16 bit patterns.

    bf16 keeps 8 significant bits.  For |v| >= 2^-126, write v = m * 2^e with
    0.5 <= |m| < 1, round m * 2^8 to an integer (ties to even) and rescale; below
    2^-126 the quantum is the fixed subnormal step 2^-133.  Results of magnitude
    >= 2^128 overflow to +-inf; NaN stays NaN.  The rounded value is exactly
    representable in fp32, whose top 16 bits are the bf16 pattern.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    y = np.ldexp(np.rint(m * 256.0), e - 8)
    tiny = np.abs(v) < 2.0 ** -126
    y = np.where(tiny, np.rint(v * 2.0 ** 133) * 2.0 ** -133, y)
    big = np.abs(y) >= 2.0 ** 128
    y = np.where(big, np.copysign(np.inf, v), y)
    y = np.where(np.isnan(v), np.nan, y)
    f32 = y.astype(np.float32)
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(v), np.uint16(0x7FC0), bits).astype(np.uint16)
    return bits


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x|: 2^(floor(log2|x|) - 7), 2^-133 below 2^-126."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    u = np.ldexp(1.0, (e - 7).astype(np.int64))
    return np.where(a < 2.0 ** -126, 2.0 ** -133, u)


# ---------------------------------------------------------------------------
# 2.-3. The grouped contraction with factored scales.
# ---------------------------------------------------------------------------

def _accumulate(a_codes: np.ndarray, b_codes: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k dec(a[m, k]) * dec(b[n, k]) in fp64 (exact, see header)."""
    a = decode_e4m3fn(a_codes)
    b = decode_e4m3fn(b_codes)
    return a @ b.T


def _apply_scales(acc: np.ndarray, xs: np.ndarray, ws: np.ndarray) -> np.ndarray:
    """(acc * x_scale[m]) * w_scale[n], fp32 scales widened exactly to fp64."""
    return (acc * np.asarray(xs, np.float64)[:, None]) * np.asarray(ws, np.float64)[None, :]


@dataclass
class OracleResult:
    """values: fp64 result before rounding (NaN where the row is not written),
    bits: bf16 patterns (0 in zeroed rows, 0x7FC1 where untouched),
    row_class: per output row, one of ROW_WRITTEN / ROW_ZEROED / ROW_UNTOUCHED."""

    values: np.ndarray
    bits: np.ndarray
    row_class: np.ndarray
    col_class: np.ndarray | None = None   # n_offsets: per output column (else None)

    def written_values_rounded(self) -> np.ndarray:
        return bf16_bits_to_f64(self.bits[self.row_class == ROW_WRITTEN])


UNTOUCHED_SENTINEL = np.uint16(0x7FC1)


def stacked_row_groups(M_sizes: np.ndarray, total_M: int) -> np.ndarray:
    """Owning group of each stacked row, or -1 for rows that belong to none.

    Group g owns rows [start_g, start_g + max(M_sizes[g], 0)) with start_g the
    running sum of the (clamped) sizes before it, cut at total_M.
    """
    sizes = np.clip(np.asarray(M_sizes, dtype=np.int64), 0, None)
    owner = np.full(int(total_M), -1, dtype=np.int64)
    start = 0
    for g, s in enumerate(sizes.tolist()):
        lo = min(start, total_M)
        hi = min(start + s, total_M)
        owner[lo:hi] = g
        start += s
    return owner


def offsets_row_groups(offsets: np.ndarray, total_M: int) -> np.ndarray:
    """Owning group of each row of the offsets layout, or -1 for rows of none.

    Group g owns rows [end_{g-1}, end_g), end_{-1} = 0, with
    end_g = min(max(offsets[g], end_{g-1}), total_M).
    """
    owner = np.full(int(total_M), -1, dtype=np.int64)
    prev = 0
    for g, o in enumerate(np.asarray(offsets, dtype=np.int64).tolist()):
        end = min(max(o, prev), total_M)
        owner[prev:end] = g
        prev = end
    return owner


def grouped_stacked(XQ, WQ, x_scale, w_scale, M_sizes) -> OracleResult:
    """Stacked layout: XQ [total_M, K], WQ [G, N, K], x_scale [total_M],
    w_scale [G, N], M_sizes [G] -> Y [total_M, N]."""
    XQ = np.asarray(XQ, np.uint8)
    return _grouped_packed(XQ, WQ, x_scale, w_scale, stacked_row_groups(M_sizes, XQ.shape[0]))


def grouped_offsets(XQ, WQ, x_scale, w_scale, offsets) -> OracleResult:
    """Offsets layout: XQ [total_M, K], WQ [G, N, K], x_scale [total_M],
    w_scale [G, N], offsets [G] int32 inclusive prefix -> Y [total_M, N]."""
    XQ = np.asarray(XQ, np.uint8)
    return _grouped_packed(XQ, WQ, x_scale, w_scale, offsets_row_groups(offsets, XQ.shape[0]))


def _grouped_packed(XQ, WQ, x_scale, w_scale, owner) -> OracleResult:
    """Groups packed along M; owner[r] is the group of row r (-1: none)."""
    XQ = np.asarray(XQ, np.uint8)
    WQ = np.asarray(WQ, np.uint8)
    total_M, K = XQ.shape
    G, N, K2 = WQ.shape
    assert K == K2
    values = np.full((total_M, N), np.nan)
    bits = np.full((total_M, N), UNTOUCHED_SENTINEL, dtype=np.uint16)
    row_class = np.full(total_M, ROW_UNTOUCHED, dtype=np.int8)
    if K == 0:
        values[:] = 0.0
        bits[:] = 0
        row_class[:] = ROW_ZEROED
        return OracleResult(values, bits, row_class)
    for g in range(G):
        rows = np.nonzero(owner == g)[0]
        if rows.size == 0:
            continue
        acc = _accumulate(XQ[rows], WQ[g])
        v = _apply_scales(acc, np.asarray(x_scale)[rows], np.asarray(w_scale)[g])
        values[rows] = v
        bits[rows] = bf16_rne_from_f64(v)
        row_class[rows] = ROW_WRITTEN
    return OracleResult(values, bits, row_class)


def dynamic_row_classes(zero_start_index_M, expected_m: int, zeroing: bool = True) -> np.ndarray:
    """Row classes [G, expected_m] of the padded layout."""
    z = np.clip(np.asarray(zero_start_index_M, np.int64), 0, expected_m)
    i = np.arange(expected_m)[None, :]
    pad = ROW_ZEROED if zeroing else ROW_UNTOUCHED
    return np.where(i < z[:, None], ROW_WRITTEN, pad).astype(np.int8)


def grouped_dynamic(XQ, WQ, x_scale, w_scale, zero_start_index_M,
                    zeroing_output_tensor: bool = True) -> OracleResult:
    """Padded layout: XQ [G, em, K], WQ [G, N, K], x_scale [G, em], w_scale [G, N],
    zero_start_index_M [G] -> Y [G, em, N] (flattened row classes [G*em])."""
    XQ = np.asarray(XQ, np.uint8)
    WQ = np.asarray(WQ, np.uint8)
    G, em, K = XQ.shape
    G2, N, K2 = WQ.shape
    assert G == G2 and K == K2
    values = np.full((G, em, N), np.nan)
    bits = np.full((G, em, N), UNTOUCHED_SENTINEL, dtype=np.uint16)
    if K == 0:
        values[:] = 0.0
        bits[:] = 0
        return OracleResult(values, bits, np.full(G * em, ROW_ZEROED, np.int8))
    cls = dynamic_row_classes(zero_start_index_M, em, zeroing_output_tensor)
    for g in range(G):
        valid = np.nonzero(cls[g] == ROW_WRITTEN)[0]
        if valid.size:
            acc = _accumulate(XQ[g, valid], WQ[g])
            v = _apply_scales(acc, np.asarray(x_scale)[g, valid], np.asarray(w_scale)[g])
            values[g, valid] = v
            bits[g, valid] = bf16_rne_from_f64(v)
        zeroed = cls[g] == ROW_ZEROED
        values[g, zeroed] = 0.0
        bits[g, zeroed] = 0
    return OracleResult(values, bits, cls.reshape(-1))


def grouped_batched(XQ, WQ, x_scale, w_scale) -> OracleResult:
    """Batched layout: XQ [G, M, K], WQ [G, N, K], x_scale [G, M], w_scale [G, N]
    -> Y [G, M, N], every row written (flattened row classes [G*M])."""
    XQ = np.asarray(XQ, np.uint8)
    WQ = np.asarray(WQ, np.uint8)
    G, M, K = XQ.shape
    G2, N, K2 = WQ.shape
    assert G == G2 and K == K2
    if K == 0:
        return OracleResult(np.zeros((G, M, N)), np.zeros((G, M, N), np.uint16),
                            np.full(G * M, ROW_ZEROED, np.int8))
    values = np.empty((G, M, N))
    for g in range(G):
        acc = _accumulate(XQ[g], WQ[g])
        values[g] = _apply_scales(acc, np.asarray(x_scale)[g], np.asarray(w_scale)[g])
    return OracleResult(values, bf16_rne_from_f64(values), np.full(G * M, ROW_WRITTEN, np.int8))


def n_offsets_col_groups(n_offsets: np.ndarray, total_N: int) -> np.ndarray:
    """Owning group of each output column of the n_offsets layout, or -1.

    Group g owns columns [end_{g-1}, end_g), end_{-1} = 0, with
    end_g = min(max(n_offsets[g], end_{g-1}), total_N).
    """
    owner = np.full(int(total_N), -1, dtype=np.int64)
    prev = 0
    for g, o in enumerate(np.asarray(n_offsets, dtype=np.int64).tolist()):
        end = min(max(o, prev), total_N)
        owner[prev:end] = g
        prev = end
    return owner


def grouped_n_offsets(XQ, WQ, x_scale, w_scale, n_offsets) -> OracleResult:
    """N-offsets layout (3D-2D): XQ [G, M, K], WQ [total_N, K], x_scale [G, M],
    w_scale [total_N], n_offsets [G] int32 inclusive prefix over W's rows
    -> Y [M, total_N].  Column n of group g:
        Y[m, n] = (sum_k dec(XQ[g, m, k]) dec(WQ[n, k])) * x_scale[g, m] * w_scale[n].
    Columns of no group are untouched (col_class)."""
    XQ = np.asarray(XQ, np.uint8)
    WQ = np.asarray(WQ, np.uint8)
    G, M, K = XQ.shape
    total_N, K2 = WQ.shape
    assert K == K2
    values = np.full((M, total_N), np.nan)
    bits = np.full((M, total_N), UNTOUCHED_SENTINEL, dtype=np.uint16)
    col_class = np.full(total_N, ROW_UNTOUCHED, dtype=np.int8)
    if K == 0:
        return OracleResult(np.zeros((M, total_N)), np.zeros((M, total_N), np.uint16),
                            np.full(M, ROW_ZEROED, np.int8), np.full(total_N, ROW_ZEROED, np.int8))
    owner = n_offsets_col_groups(n_offsets, total_N)
    for g in range(G):
        cols = np.nonzero(owner == g)[0]
        if cols.size == 0:
            continue
        acc = _accumulate(XQ[g], WQ[cols])
        v = _apply_scales(acc, np.asarray(x_scale)[g], np.asarray(w_scale)[cols])
        values[:, cols] = v
        bits[:, cols] = bf16_rne_from_f64(v)
        col_class[cols] = ROW_WRITTEN
    row_class = np.full(M, ROW_WRITTEN if np.any(col_class == ROW_WRITTEN) else ROW_UNTOUCHED, np.int8)
    return OracleResult(values, bits, row_class, col_class)


def k_offsets_slices(k_offsets: np.ndarray, total_K: int) -> list:
    """K slice [start, end) of each group of the k_offsets layout: end_g =
    min(max(k_offsets[g], end_{g-1}), total_K), start_g = end_{g-1}, end_{-1} = 0."""
    out = []
    prev = 0
    for o in np.asarray(k_offsets, dtype=np.int64).tolist():
        end = min(max(o, prev), total_K)
        out.append((prev, end))
        prev = end
    return out


def grouped_k_offsets(XQ, WQ, x_scale, w_scale, k_offsets) -> OracleResult:
    """K-offsets layout (2D-2D): XQ [M, total_K], WQ [N, total_K], x_scale [G, M],
    w_scale [G, N], k_offsets [G] int32 inclusive prefix over K -> Y [G, M, N]:
        Y[g, m, n] = (sum_{k in slice g} dec(XQ[m, k]) dec(WQ[n, k])) * x_scale[g, m] * w_scale[g, n].
    Every row of every group is written (flattened row classes [G*M])."""
    XQ = np.asarray(XQ, np.uint8)
    WQ = np.asarray(WQ, np.uint8)
    M, total_K = XQ.shape
    N, K2 = WQ.shape
    assert total_K == K2
    slices = k_offsets_slices(k_offsets, total_K)
    G = len(slices)
    if total_K == 0:
        return OracleResult(np.zeros((G, M, N)), np.zeros((G, M, N), np.uint16),
                            np.full(G * M, ROW_ZEROED, np.int8))
    values = np.empty((G, M, N))
    for g, (ks, ke) in enumerate(slices):
        acc = _accumulate(XQ[:, ks:ke], WQ[:, ks:ke])
        values[g] = _apply_scales(acc, np.asarray(x_scale)[g], np.asarray(w_scale)[g])
    return OracleResult(values, bf16_rne_from_f64(values), np.full(G * M, ROW_WRITTEN, np.int8))


# ---------------------------------------------------------------------------
# Sampled outputs for full-size problems (same arithmetic, chosen entries only).
# ---------------------------------------------------------------------------

def stacked_entries(XQ, WQ, x_scale, w_scale, M_sizes, rows, cols):
    """Oracle values (fp64) and bf16 bits at Y[rows[i], cols[j]] for every i, j.

    Rows owned by no group come back as NaN / the untouched sentinel.
    Returns (values [len(rows), len(cols)], bits, owner_of_rows).
    """
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    total_M = np.asarray(XQ).shape[0]
    owner = stacked_row_groups(M_sizes, total_M)[rows]
    values = np.full((rows.size, cols.size), np.nan)
    for g in np.unique(owner[owner >= 0]):
        sel = np.nonzero(owner == g)[0]
        acc = _accumulate(np.asarray(XQ)[rows[sel]], np.asarray(WQ)[g][cols])
        values[sel] = _apply_scales(acc, np.asarray(x_scale)[rows[sel]],
                                    np.asarray(w_scale)[g][cols])
    bits = np.where(np.isnan(values), UNTOUCHED_SENTINEL, bf16_rne_from_f64(values))
    return values, bits.astype(np.uint16), owner


def dynamic_entries(XQ, WQ, x_scale, w_scale, zero_start_index_M, groups, rows, cols):
    """Oracle values at Y[groups[i], rows[i], cols[j]] (valid rows only; padding
    rows come back as exact zeros).  Returns (values, bits, row_class)."""
    groups = np.asarray(groups, np.int64)
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    em = np.asarray(XQ).shape[1]
    cls = dynamic_row_classes(zero_start_index_M, em, True)[groups, rows]
    values = np.zeros((rows.size, cols.size))
    for g in np.unique(groups):
        sel = np.nonzero((groups == g) & (cls == ROW_WRITTEN))[0]
        if sel.size == 0:
            continue
        acc = _accumulate(np.asarray(XQ)[g, rows[sel]], np.asarray(WQ)[g][cols])
        values[sel] = _apply_scales(acc, np.asarray(x_scale)[g, rows[sel]],
                                    np.asarray(w_scale)[g][cols])
    return values, bf16_rne_from_f64(values), cls
