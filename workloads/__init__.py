"""Seeded synthetic inputs for the FP8 rowwise-scaled grouped GEMM.

This module only draws inputs: group metadata, normal values, and their rowwise
fp8 (e4m3fn) quantisation with fp32 scales.  It holds none of the grouped GEMM's
arithmetic, so both the CPU oracle and the GPU path can take their operands from
here without sharing any code with each other.

Recipe (the same for every workload):
  * group metadata is drawn first from ``numpy.random.default_rng(seed)``;
  * values are standard normals (times ``sigma``) drawn in row chunks, chunk ``c``
    of operand ``tag`` from ``default_rng([seed, tag, c])`` so that large operands
    can be drawn on several threads and still be reproducible;
  * each row (of XQ, and of WQ[g] for each output column n) is quantised on its own:
    ``s = amax / 448`` in fp32 (``s = 1`` for an all-zero row), ``q = e4m3fn(clamp(x / s,
    -448, 448))`` with round-to-nearest-even.  The clamp comes before the cast
    because torch's float8 cast does not saturate.

The fp8 cast is torch's CPU ``float8_e4m3fn`` conversion; everything else is numpy.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

E4M3_MAX = 448.0
_CHUNK_ELEMS = 1 << 24  # elements per drawn chunk (keeps transient fp32 memory small)

_TAG_X = 1
_TAG_W = 2


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cast_e4m3fn(x: np.ndarray) -> np.ndarray:
    """fp32 -> e4m3fn bytes (round to nearest even) via torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Rowwise fp8 quantisation of a float32 ``[..., K]`` array.

    Returns (q, s): ``q`` uint8 e4m3fn codes of x's shape, ``s`` float32 of shape
    ``x.shape[:-1]`` with ``x ~= decode(q) * s``.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.shape[-1] == 0:
        return np.zeros(x.shape, np.uint8), np.ones(x.shape[:-1], np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s[s == 0] = np.float32(1.0)
    y = np.clip(x / s[..., None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return _cast_e4m3fn(y), s


def draw_quantized(seed: int, tag: int, rows: int, K: int, sigma: float = 1.0
                   ) -> tuple[np.ndarray, np.ndarray]:
    """Draw ``rows`` x ``K`` normal values and quantise them rowwise.

    Rows are drawn in chunks on a thread pool; chunk ``c`` uses
    ``default_rng([seed, tag, c])``.
    """
    q = np.empty((rows, K), np.uint8)
    s = np.empty((rows,), np.float32)
    if rows == 0 or K == 0:
        s[:] = 1.0
        q[:] = 0
        return q, s
    rows_per_chunk = max(1, _CHUNK_ELEMS // K)
    starts = list(range(0, rows, rows_per_chunk))

    def work(ci: int) -> None:
        r0 = starts[ci]
        r1 = min(rows, r0 + rows_per_chunk)
        rng = np.random.default_rng([seed, tag, ci])
        x = rng.standard_normal((r1 - r0, K), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        q[r0:r1], s[r0:r1] = quantize_rows(x)

    if len(starts) == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(len(starts))))
    return q, s


@dataclass
class Stacked:
    """Inputs of the stacked layout: groups concatenated along M."""

    XQ: np.ndarray        # [total_M, K] uint8 (e4m3fn codes)
    WQ: np.ndarray        # [G, N, K] uint8
    x_scale: np.ndarray   # [total_M] float32
    w_scale: np.ndarray   # [G, N] float32
    M_sizes: np.ndarray   # [G] int64
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return int(self.WQ.shape[0])

    @property
    def N(self) -> int:
        return int(self.WQ.shape[1])

    @property
    def K(self) -> int:
        return int(self.WQ.shape[2])

    @property
    def total_M(self) -> int:
        return int(self.XQ.shape[0])


@dataclass
class Dynamic:
    """Inputs of the padded ("dynamic") layout: one expected_m slab per group."""

    XQ: np.ndarray                  # [G, expected_m, K] uint8
    WQ: np.ndarray                  # [G, N, K] uint8
    x_scale: np.ndarray             # [G, expected_m] float32
    w_scale: np.ndarray             # [G, N] float32
    zero_start_index_M: np.ndarray  # [G] int64
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return int(self.WQ.shape[0])

    @property
    def N(self) -> int:
        return int(self.WQ.shape[1])

    @property
    def K(self) -> int:
        return int(self.WQ.shape[2])

    @property
    def expected_m(self) -> int:
        return int(self.XQ.shape[1])


def make_stacked(M_sizes, N: int, K: int, seed: int, sigma: float = 1.0,
                 total_M: int | None = None, name: str = "") -> Stacked:
    """Stacked-layout inputs for the given per-group row counts.

    ``total_M`` defaults to ``sum(M_sizes)``; a larger value leaves trailing rows
    that belong to no group.
    """
    M_sizes = np.asarray(M_sizes, dtype=np.int64)
    G = int(M_sizes.shape[0])
    if total_M is None:
        total_M = int(np.clip(M_sizes, 0, None).sum())
    XQ, xs = draw_quantized(seed, _TAG_X, total_M, K, sigma)
    WQ, ws = draw_quantized(seed, _TAG_W, G * N, K, sigma)
    return Stacked(XQ, WQ.reshape(G, N, K), xs, ws.reshape(G, N), M_sizes, name)


def make_dynamic(zero_start_index_M, expected_m: int, N: int, K: int, seed: int,
                 sigma: float = 1.0, name: str = "") -> Dynamic:
    """Padded-layout inputs.  Every row of every slab is drawn, padding included."""
    zsi = np.asarray(zero_start_index_M, dtype=np.int64)
    G = int(zsi.shape[0])
    XQ, xs = draw_quantized(seed, _TAG_X, G * expected_m, K, sigma)
    WQ, ws = draw_quantized(seed, _TAG_W, G * N, K, sigma)
    return Dynamic(XQ.reshape(G, expected_m, K), WQ.reshape(G, N, K),
                   xs.reshape(G, expected_m), ws.reshape(G, N), zsi, name)


# ---------------------------------------------------------------------------
# The five MoE-shaped workloads.
# ---------------------------------------------------------------------------

DOWN_PROJ_TOTAL_M = (1, 8, 32, 256, 2048, 8192)


def zipf_sizes(seed: int, total: int, G: int, exponent: float = 1.2) -> np.ndarray:
    """Zipf-shaped token split with one group forced empty.

    Rank weights r^-exponent are assigned to groups by a seeded permutation; the
    group that receives the last rank gets weight 0; counts are one multinomial draw.
    """
    rng = np.random.default_rng(seed)
    w = np.arange(1, G + 1, dtype=np.float64) ** (-exponent)
    perm = rng.permutation(G)
    p = np.empty(G)
    p[perm] = w
    p[perm[-1]] = 0.0
    p /= p.sum()
    return rng.multinomial(total, p).astype(np.int64)


def uniform_sizes(seed: int, total: int, G: int) -> np.ndarray:
    """Each token goes to a group drawn uniformly at random."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, G, size=total)
    return np.bincount(ids, minlength=G).astype(np.int64)


def padded_valid_rows(seed: int, G: int, expected_m: int) -> np.ndarray:
    """Uniform valid-row counts in [0, expected_m], group 0 empty, group 1 full."""
    rng = np.random.default_rng(seed)
    z = rng.integers(0, expected_m + 1, G)
    z[0] = 0
    z[1] = expected_m
    return z.astype(np.int64)


def tiny_stacked() -> Stacked:
    """G=4, M_sizes={0,3,17,44}, N=256, K=512."""
    return make_stacked([0, 3, 17, 44], 256, 512, seed=1001, name="tiny_stacked_G4_M64_N256_K512")


def moe_gate_up() -> Stacked:
    """G=8, total_M=4096 split by Zipf(1.2) with one empty group, N=4096, K=7168."""
    sizes = zipf_sizes(2002, 4096, 8)
    return make_stacked(sizes, 4096, 7168, seed=2002, name="moe_gate_up_G8_M4096_N4096_K7168")


def moe_down(total_M: int) -> Stacked:
    """G=8, tokens spread uniformly over groups, N=7168, K=2048."""
    sizes = uniform_sizes(3000 + total_M, total_M, 8)
    return make_stacked(sizes, 7168, 2048, seed=3000 + total_M,
                        name=f"moe_down_G8_M{total_M}_N7168_K2048")


def dense_expert() -> Stacked:
    """G=4, 512 rows per group, N=8192, K=28672, values N(0, 0.5)."""
    return make_stacked([512] * 4, 8192, 28672, seed=4004, sigma=0.5,
                        name="dense_expert_G4_M2048_N8192_K28672")


def padded_tails() -> Dynamic:
    """G=16, expected_m=512, N=1000, K=7184 (tails on N and K)."""
    z = padded_valid_rows(5005, 16, 512)
    return make_dynamic(z, 512, 1000, 7184, seed=5005, name="padded_G16_em512_N1000_K7184")


def gen_rows_from(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Seeded integers in [lo, hi) (helper for randomised edge cases)."""
    return np.random.default_rng(seed).integers(lo, hi, n).astype(np.int64)


# ---------------------------------------------------------------------------
# Layouts whose groups partition N (n_offsets, 3D-2D) or K (k_offsets, 2D-2D).
# ---------------------------------------------------------------------------

@dataclass
class NOffsets:
    """Inputs of the n_offsets layout: one X slab per group, W rows split by group."""
    XQ: np.ndarray         # [G, M, K] uint8
    WQ: np.ndarray         # [total_N, K] uint8
    x_scale: np.ndarray    # [G, M] float32
    w_scale: np.ndarray    # [total_N] float32
    n_offsets: np.ndarray  # [G] int32 inclusive prefix of the group widths
    name: str = ""

    @property
    def G(self) -> int:
        return int(self.XQ.shape[0])

    @property
    def M(self) -> int:
        return int(self.XQ.shape[1])

    @property
    def N(self) -> int:
        return int(self.WQ.shape[0])

    @property
    def K(self) -> int:
        return int(self.WQ.shape[1])


@dataclass
class KOffsets:
    """Inputs of the k_offsets layout: both operands split along K by group; each
    group's slice of a row is quantised on its own (one scale per group and row)."""
    XQ: np.ndarray         # [M, total_K] uint8
    WQ: np.ndarray         # [N, total_K] uint8
    x_scale: np.ndarray    # [G, M] float32
    w_scale: np.ndarray    # [G, N] float32
    k_offsets: np.ndarray  # [G] int32 inclusive prefix of the slice lengths
    name: str = ""

    @property
    def G(self) -> int:
        return int(self.k_offsets.shape[0])

    @property
    def M(self) -> int:
        return int(self.XQ.shape[0])

    @property
    def N(self) -> int:
        return int(self.WQ.shape[0])

    @property
    def K(self) -> int:
        return int(self.XQ.shape[1])


def make_n_offsets(widths, M: int, K: int, seed: int, total_N: int | None = None, sigma: float = 1.0,
                   name: str = "") -> NOffsets:
    """n_offsets inputs for the given group widths (columns per group); ``total_N``
    larger than their sum leaves trailing columns that belong to no group."""
    widths = np.asarray(widths, dtype=np.int64)
    G = int(widths.shape[0])
    if total_N is None:
        total_N = int(widths.sum())
    XQ, xs = draw_quantized(seed, _TAG_X, G * M, K, sigma)
    WQ, ws = draw_quantized(seed, _TAG_W, total_N, K, sigma)
    return NOffsets(XQ.reshape(G, M, K), WQ, xs.reshape(G, M), ws, np.cumsum(widths).astype(np.int32), name)


def _quantize_slices(x: np.ndarray, bounds) -> tuple[np.ndarray, np.ndarray]:
    """Rowwise quantisation of each K slice [ks, ke) of x [rows, K] on its own:
    codes [rows, K] (columns past the last slice quantised as one more slice)
    and scales [G, rows]."""
    rows, K = x.shape
    q = np.zeros((rows, K), np.uint8)
    s = np.ones((len(bounds), rows), np.float32)
    for g, (ks, ke) in enumerate(bounds):
        q[:, ks:ke], s[g] = quantize_rows(x[:, ks:ke])
    last = bounds[-1][1] if bounds else 0
    if last < K:
        q[:, last:], _ = quantize_rows(x[:, last:])
    return q, s


def make_k_offsets(lengths, M: int, N: int, seed: int, total_K: int | None = None, sigma: float = 1.0,
                   name: str = "") -> KOffsets:
    """k_offsets inputs for the given slice lengths (K bytes per group)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    if total_K is None:
        total_K = int(lengths.sum())
    ends = np.cumsum(lengths)
    bounds = [(int(e - n), int(e)) for e, n in zip(ends, lengths)]
    rx = np.random.default_rng([seed, _TAG_X])
    rw = np.random.default_rng([seed, _TAG_W])
    x = rx.standard_normal((M, total_K), dtype=np.float32) * np.float32(sigma)
    w = rw.standard_normal((N, total_K), dtype=np.float32) * np.float32(sigma)
    XQ, xs = _quantize_slices(x, bounds)
    del x
    WQ, ws = _quantize_slices(w, bounds)
    return KOffsets(XQ, WQ, xs, ws, ends.astype(np.int32), name)


def moe_n_offsets() -> NOffsets:
    """G=8 slabs of M=512 rows, K=7168; 16384 weight rows split over the groups by
    Zipf(1.2) in units of 8 columns, one group empty."""
    widths = 8 * zipf_sizes(6006, 2048, 8)
    return make_n_offsets(widths, 512, 7168, seed=6006, name="moe_n_offsets_G8_M512_N16384_K7168")


def moe_wgrad_k_offsets() -> KOffsets:
    """Weight-gradient shape: G=8 groups slicing 4096 tokens of K by Zipf(1.2) in
    units of 16, one group empty; M=2048, N=7168, Y [8, 2048, 7168]."""
    lengths = 16 * zipf_sizes(7007, 256, 8)
    return make_k_offsets(lengths, 2048, 7168, seed=7007, name="moe_wgrad_k_offsets_G8_M2048_N7168_K4096")


# ---------------------------------------------------------------------------
# Block (groupwise) scales: one scale per (row, K block) of X and per
# (block_n rows, K block) block of each W[g].
# ---------------------------------------------------------------------------

@dataclass
class StackedBlockscale:
    XQ: np.ndarray        # [total_M, K] uint8
    WQ: np.ndarray        # [G, N, K] uint8
    x_scale: np.ndarray   # [total_M, K / block_k] float32
    w_scale: np.ndarray   # [G, N / block_n, K / block_k] float32
    M_sizes: np.ndarray   # [G] int64
    block_k: int = 128
    block_n: int = 128
    name: str = ""

    @property
    def G(self) -> int:
        return int(self.WQ.shape[0])

    @property
    def N(self) -> int:
        return int(self.WQ.shape[1])

    @property
    def K(self) -> int:
        return int(self.WQ.shape[2])

    @property
    def total_M(self) -> int:
        return int(self.XQ.shape[0])


def quantize_blocks(x: np.ndarray, rows_per_block: int, block_k: int) -> tuple[np.ndarray, np.ndarray]:
    """Blockwise fp8 quantisation of a float32 [R, K] array: one scale per
    (rows_per_block x block_k) block (amax / 448, 1 for an all-zero block), the
    same clamp-then-cast as quantize_rows.  Returns (codes [R, K], scales
    [R / rows_per_block, K / block_k])."""
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    xb = x.reshape(R // rows_per_block, rows_per_block, K // block_k, block_k)
    amax = np.max(np.abs(xb), axis=(1, 3))
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s[s == 0] = np.float32(1.0)
    y = np.clip(xb / s[:, None, :, None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return _cast_e4m3fn(y.reshape(R, K)), s


def make_stacked_blockscale(M_sizes, N: int, K: int, seed: int, sigma: float = 1.0, block_k: int = 128,
                            block_n: int = 128, total_M: int | None = None, name: str = "") -> StackedBlockscale:
    """Stacked inputs with block scales; values drawn as for make_stacked (row chunks
    per operand), then quantised per block."""
    M_sizes = np.asarray(M_sizes, dtype=np.int64)
    G = int(M_sizes.shape[0])
    if total_M is None:
        total_M = int(np.clip(M_sizes, 0, None).sum())
    rx = np.random.default_rng([seed, _TAG_X])
    x = rx.standard_normal((total_M, K), dtype=np.float32) * np.float32(sigma)
    XQ, xs = quantize_blocks(x, 1, block_k)
    del x
    WQ = np.empty((G, N, K), np.uint8)
    ws = np.empty((G, N // block_n, K // block_k), np.float32)
    for g in range(G):
        rw = np.random.default_rng([seed, _TAG_W, g])
        w = rw.standard_normal((N, K), dtype=np.float32) * np.float32(sigma)
        WQ[g], ws[g] = quantize_blocks(w, block_n, block_k)
    return StackedBlockscale(XQ, WQ, xs, ws, M_sizes, block_k, block_n, name)


def moe_gate_up_blockscale() -> StackedBlockscale:
    """The gate_up shape (G=8, Zipf(1.2) split of 4096 rows, N=4096, K=7168) with
    128 x 128 weight blocks and 1 x 128 activation blocks."""
    sizes = zipf_sizes(2002, 4096, 8)
    return make_stacked_blockscale(sizes, 4096, 7168, seed=8008, name="moe_gate_up_blockscale_G8_M4096_N4096_K7168")


def make_dynamic_blockscale(zero_start_index_M, expected_m: int, N: int, K: int, seed: int, sigma: float = 1.0,
                            name: str = "") -> Dynamic:
    """Padded-layout inputs with block scales: every slab row drawn, X quantised per
    (row, 128) block (x_scale [G, expected_m, K/128]) and each W[g] per 128 x 128
    block (w_scale [G, N/128, K/128])."""
    zsi = np.asarray(zero_start_index_M, dtype=np.int64)
    G = int(zsi.shape[0])
    w = make_stacked_blockscale([expected_m] * G, N, K, seed, sigma)
    return Dynamic(w.XQ.reshape(G, expected_m, K), w.WQ, w.x_scale.reshape(G, expected_m, K // 128), w.w_scale,
                   zsi, name)


def padded_blockscale() -> Dynamic:
    """The padded workload's slabs and valid rows (G=16, expected_m=512) with block
    scales, at N=1024, K=7168 (whole 128-wide blocks)."""
    z = padded_valid_rows(5005, 16, 512)
    return make_dynamic_blockscale(z, 512, 1024, 7168, seed=9009, name="padded_blockscale_G16_em512_N1024_K7168")
