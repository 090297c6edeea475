"""Exact rational brute force for tiny grouped GEMMs (a pin for the oracle).

Independent of ``oracle/``: fp8 codes are decoded by torch's own float8_e4m3fn
type, every product and sum is an exact ``Fraction``, and bf16 rounding is done
on the exact rational with round-half-to-even.  Pure Python loops: tiny shapes only.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch


def torch_decode_all() -> list:
    """Exact value of every e4m3fn code as decoded by torch (None for NaN)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float32).tolist()
    return [None if v != v else Fraction(v) for v in vals]


_DEC = torch_decode_all()


def bf16_bits_exact(v) -> int:
    """Round an exact rational (or None = NaN) to bf16 with ties-to-even."""
    if v is None:
        return 0x7FC0
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    # e = floor(log2(a))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (-133) if e < -126 else Fraction(2) ** (e - 7)
    q = a / quantum
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    y = n * quantum
    if y >= Fraction(2) ** 128:
        return sign | 0x7F80
    f = np.float32(float(y))  # exact: y has <= 8 significant bits in range
    assert Fraction(float(f)) == y
    return sign | int(f.view(np.uint32) >> np.uint32(16))


def dot_exact(a_codes, b_codes):
    acc = Fraction(0)
    for x, w in zip(a_codes.tolist(), b_codes.tolist()):
        dx, dw = _DEC[x], _DEC[w]
        if dx is None or dw is None:
            return None
        acc += dx * dw
    return acc


def stacked_exact(XQ, WQ, x_scale, w_scale, M_sizes):
    """Exact bf16 bits [total_M, N]; rows of no group are None."""
    total_M = XQ.shape[0]
    G, N, _ = WQ.shape
    out = [None] * total_M
    start = 0
    for g in range(G):
        s = max(int(M_sizes[g]), 0)
        for r in range(start, min(start + s, total_M)):
            row = []
            for n in range(N):
                acc = dot_exact(XQ[r], WQ[g, n])
                v = None if acc is None else acc * Fraction(float(x_scale[r])) * Fraction(float(w_scale[g, n]))
                row.append(bf16_bits_exact(v))
            out[r] = row
        start += s
    return out


def offsets_exact(XQ, WQ, x_scale, w_scale, offsets):
    """Exact bf16 bits [total_M, N] for well-formed offsets (non-decreasing, at most
    total_M): group g owns rows offsets[g-1] .. offsets[g]-1, offsets[-1] = 0."""
    total_M = XQ.shape[0]
    G, N, _ = WQ.shape
    out = [None] * total_M
    for g in range(G):
        lo = int(offsets[g - 1]) if g > 0 else 0
        for r in range(lo, int(offsets[g])):
            row = []
            for n in range(N):
                acc = dot_exact(XQ[r], WQ[g, n])
                v = None if acc is None else acc * Fraction(float(x_scale[r])) * Fraction(float(w_scale[g, n]))
                row.append(bf16_bits_exact(v))
            out[r] = row
    return out


def n_offsets_exact(XQ, WQ, x_scale, w_scale, n_offsets):
    """Exact bf16 bits [M][total_N] of the n_offsets (3D-2D) layout for well-formed
    offsets: group g owns W rows (output columns) n_offsets[g-1] .. n_offsets[g]-1,
    n_offsets[-1] = 0, and multiplies them against its slab XQ[g].  Columns of no
    group are None."""
    G, M, _ = XQ.shape
    total_N = WQ.shape[0]
    out = [[None] * total_N for _ in range(M)]
    for g in range(G):
        lo = int(n_offsets[g - 1]) if g > 0 else 0
        for n in range(lo, int(n_offsets[g])):
            for m in range(M):
                acc = dot_exact(XQ[g, m], WQ[n])
                v = None if acc is None else acc * Fraction(float(x_scale[g, m])) * Fraction(float(w_scale[n]))
                out[m][n] = bf16_bits_exact(v)
    return out


def k_offsets_exact(XQ, WQ, x_scale, w_scale, k_offsets):
    """Exact bf16 bits [G][M][N] of the k_offsets (2D-2D) layout for well-formed
    offsets: group g contracts over K columns k_offsets[g-1] .. k_offsets[g]-1 of
    both operands, k_offsets[-1] = 0."""
    M = XQ.shape[0]
    N = WQ.shape[0]
    out = []
    for g in range(len(k_offsets)):
        lo = int(k_offsets[g - 1]) if g > 0 else 0
        hi = int(k_offsets[g])
        slab = []
        for m in range(M):
            row = []
            for n in range(N):
                acc = dot_exact(XQ[m, lo:hi], WQ[n, lo:hi])
                v = None if acc is None else acc * Fraction(float(x_scale[g, m])) * Fraction(float(w_scale[g, n]))
                row.append(bf16_bits_exact(v))
            slab.append(row)
        out.append(slab)
    return out


def blockscale_exact(XQ, WQ, x_scale, w_scale, M_sizes, block_k, block_n):
    """Exact bf16 bits [total_M][N] of the stacked layout with block scales: group
    g's row r, column n is sum over K blocks kb of (exact block dot product) *
    x_scale[r, kb] * w_scale[g, n // block_n, kb], rounded once.  Rows of no group
    are None."""
    total_M, K = XQ.shape
    G, N, _ = WQ.shape
    out = [None] * total_M
    start = 0
    for g in range(G):
        s = max(int(M_sizes[g]), 0)
        for r in range(start, min(start + s, total_M)):
            row = []
            for n in range(N):
                acc = Fraction(0)
                for kb in range(K // block_k):
                    d = dot_exact(XQ[r, kb * block_k:(kb + 1) * block_k], WQ[g, n, kb * block_k:(kb + 1) * block_k])
                    acc += d * Fraction(float(x_scale[r, kb])) * Fraction(float(w_scale[g, n // block_n, kb]))
                row.append(bf16_bits_exact(acc))
            out[r] = row
        start += s
    return out
