"""Helpers for comparing the GPU library with the CPU oracle.

Parity rule (written here, used by every GPU test):
  * row classification is bit-exact: rows the oracle writes are written, rows it
    zeroes hold +-0, rows it leaves untouched still hold the sentinel;
  * written values: |y - ref| <= 2 * ulp_bf16(|ref|) + 1e-3 * rms(ref) per element,
    ref = the oracle's bf16 result, rms over every written element of the call;
  * guard bands before and after the output keep the sentinel (no stray writes).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

SENTINEL = 0x7FC1          # a bf16 NaN pattern the kernels never produce
GUARD = 256                # bf16 elements of guard band on each side (512 bytes)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def guarded_output(shape) -> tuple[torch.Tensor, torch.Tensor]:
    """A sentinel-filled bf16 buffer with guard bands; returns (whole, view)."""
    n = int(np.prod(shape))
    whole = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.int16, device="cuda")
    view = whole[GUARD:GUARD + n].view(torch.bfloat16).view(*shape)
    return whole, view


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_guards(whole: torch.Tensor) -> None:
    b = bits_of(whole)
    assert np.all(b[:GUARD] == SENTINEL), "write before the output buffer"
    assert np.all(b[-GUARD:] == SENTINEL), "write past the output buffer"


def tolerance_ok(got_bits: np.ndarray, ref_bits: np.ndarray, rms: float) -> np.ndarray:
    got = oracle.bf16_bits_to_f64(got_bits)
    ref = oracle.bf16_bits_to_f64(ref_bits)
    tol = 2.0 * oracle.bf16_ulp(ref) + 1e-3 * rms
    with np.errstate(invalid="ignore"):
        return np.abs(got - ref) <= tol


def rms_of(bits: np.ndarray) -> float:
    v = oracle.bf16_bits_to_f64(bits)
    return float(np.sqrt(np.mean(v * v))) if v.size else 0.0


def assert_rows_match(got: np.ndarray, res: oracle.OracleResult, rms: float | None = None, label: str = "") -> None:
    """got: bf16 bits shaped [rows, N]; res: the oracle result over the same rows."""
    if res.row_class.shape[0] == 0:                 # an empty output: nothing to compare
        assert got.size == 0, f"{label}: {got.size} output elements where the oracle has none"
        return
    got = got.reshape(res.row_class.shape[0], -1)
    ref = res.bits.reshape(got.shape)
    cls = res.row_class
    w = cls == oracle.ROW_WRITTEN
    z = cls == oracle.ROW_ZEROED
    u = cls == oracle.ROW_UNTOUCHED
    if np.any(u):
        bad = np.nonzero(np.any(got[u] != SENTINEL, axis=1))[0]
        assert bad.size == 0, f"{label}: untouched rows were written: {np.nonzero(u)[0][bad][:10]}"
    if np.any(z):
        bad = np.nonzero(np.any((got[z] & 0x7FFF) != 0, axis=1))[0]
        assert bad.size == 0, f"{label}: rows that must be zero are not: {np.nonzero(z)[0][bad][:10]}"
    if np.any(w):
        gw, rw = got[w], ref[w]
        assert not np.any(gw == SENTINEL), f"{label}: written rows left unwritten"
        if rms is None:
            rms = rms_of(rw)
        ok = tolerance_ok(gw, rw, rms)
        if not np.all(ok):
            idx = np.argwhere(~ok)
            rows = np.nonzero(w)[0]
            r, c = idx[0]
            g = oracle.bf16_bits_to_f64(gw[r, c])
            e = oracle.bf16_bits_to_f64(rw[r, c])
            raise AssertionError(f"{label}: {len(idx)} elements out of tolerance; first at row {rows[r]} "
                                 f"col {c}: got {g} want {e} (rms {rms})")
