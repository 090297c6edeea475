"""GPU parity for the n_offsets (3D-2D) and k_offsets (2D-2D) layouts.

Every kernel configuration built for these layouts is forced in turn on edge
shapes (empty groups, groups narrower than a vector or a tile, group boundaries
inside a 16-byte store, K slices that end mid-stage, ill-formed prefixes) and
compared with the oracle element by element; both layouts are also compared
bitwise with the batched layout on the same products, and the two full-size
workloads are checked on sampled rows.
"""
import os
from contextlib import contextmanager

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests import parity as P

pytestmark = pytest.mark.gpu

RAGGED_CONFIGS = [2, 7, 9, 18, 21, 28]
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp8_rowwise_scaled_amd as F
    F.load()
    return F


@contextmanager
def forced(cfg):
    old = os.environ.get("FP8GG_CONFIG")
    if cfg is None:
        os.environ.pop("FP8GG_CONFIG", None)
    else:
        os.environ["FP8GG_CONFIG"] = str(cfg)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("FP8GG_CONFIG", None)
        else:
            os.environ["FP8GG_CONFIG"] = old


def _codes(rng, shape):
    return rng.choice(FINITE, size=shape).astype(np.uint8)


def _scales(rng, shape):
    return (2.0 ** rng.uniform(-10, 2, shape)).astype(np.float32)


def assert_cols_match(got, res, label=""):
    """got: bf16 bits [M, total_N]; res: the oracle's n_offsets result."""
    cls = res.col_class
    w = cls == oracle.ROW_WRITTEN
    u = cls == oracle.ROW_UNTOUCHED
    z = cls == oracle.ROW_ZEROED
    if np.any(u):
        bad = np.nonzero(np.any(got[:, u] != P.SENTINEL, axis=0))[0]
        assert bad.size == 0, f"{label}: columns of no group were written: {np.nonzero(u)[0][bad][:10]}"
    if np.any(z):
        assert np.all((got[:, z] & 0x7FFF) == 0), f"{label}: columns that must be zero are not"
    if np.any(w):
        gw, rw = got[:, w], res.bits[:, w]
        assert not np.any(gw == P.SENTINEL), f"{label}: written columns left unwritten"
        ok = P.tolerance_ok(gw, rw, P.rms_of(rw))
        if not np.all(ok):
            r, c = np.argwhere(~ok)[0]
            raise AssertionError(f"{label}: {int((~ok).sum())} elements out of tolerance; first at row {r} "
                                 f"column {np.nonzero(w)[0][c]}")


def run_n(F, XQ, WQ, xs, ws, offs):
    M, N = XQ.shape[1], WQ.shape[0]
    whole, y = P.guarded_output((M, N))
    F.f8f8bf16_rowwise_grouped_n_offsets(P.dev(XQ), P.dev(WQ), P.dev(xs), P.dev(ws),
                                         P.dev(np.asarray(offs, np.int32)), out=y)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(y)


def run_k(F, XQ, WQ, xs, ws, offs):
    G, M, N = len(offs), XQ.shape[0], WQ.shape[0]
    whole, y = P.guarded_output((G, M, N))
    F.f8f8bf16_rowwise_grouped_k_offsets(P.dev(XQ), P.dev(WQ), P.dev(xs), P.dev(ws),
                                         P.dev(np.asarray(offs, np.int32)), out=y)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(y)


# (seed, offsets, total_N, M, K); operands drawn by the workload recipe (normal
# values, rowwise-quantised), the offsets passed as given
N_CASES = [
    (101, np.cumsum([0, 1, 7, 130, 300, 64]).tolist(), 512, 37, 208),   # empty, 1, odd widths, trailing columns
    (102, [257, 264], 264, 300, 1040),                                  # two M tiles of 256, tile + 1 columns
    (103, [1000], 1000, 64, 64),                                        # one group, N tail
    (104, [40, 20, 100, 999], 96, 5, 128),                              # ill-formed: empty middle group, cut at N
    (105, np.cumsum(np.random.default_rng(7).integers(0, 40, 20)).tolist(), 400, 3, 32),  # 20 groups
]


@pytest.mark.parametrize("cfg", RAGGED_CONFIGS)
@pytest.mark.parametrize("seed,offs,total_N,M,K", N_CASES)
def test_n_offsets_matches_oracle(F, cfg, seed, offs, total_N, M, K):
    w = wl.make_n_offsets([0] * (len(offs) - 1) + [total_N], M, K, seed=seed)
    offs = np.asarray(offs, np.int32)
    res = oracle.grouped_n_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, offs)
    with forced(cfg):
        got = run_n(F, w.XQ, w.WQ, w.x_scale, w.w_scale, offs)
    assert_cols_match(got, res, f"n_offsets cfg {cfg} seed {seed}")


# (seed, k_offsets, total_K, M, N)
K_CASES = [
    (201, np.cumsum([0, 16, 48, 400, 128]).tolist(), 624, 37, 136),   # empty slice, mid-stage ends, unread tail
    (202, [1040], 1040, 300, 264),                                    # one slice, two M tiles, N tail
    (203, np.cumsum(16 * np.random.default_rng(9).integers(0, 5, 12)).tolist(), 16 * 48, 5, 64),  # 12 groups
    (204, [64, 32, 200, 99999], 160, 7, 24),                          # ill-formed: empty, cut at total_K
    (205, np.cumsum(16 * np.random.default_rng(11).integers(0, 4, 40)).tolist(), 16 * 160, 3, 40),  # 40 groups
]


@pytest.mark.parametrize("cfg", RAGGED_CONFIGS)
@pytest.mark.parametrize("seed,offs,total_K,M,N", K_CASES)
def test_k_offsets_matches_oracle(F, cfg, seed, offs, total_K, M, N):
    G = len(offs)
    # operands quantised per well-formed slice; ill-formed offsets are then passed as given
    ends = np.minimum(np.maximum.accumulate(np.maximum(np.asarray(offs, np.int64), 0)), total_K)
    w = wl.make_k_offsets(np.diff(np.concatenate([[0], ends])), M, N, seed=seed, total_K=total_K)
    offs = np.asarray(offs, np.int32)
    res = oracle.grouped_k_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, offs)
    with forced(cfg):
        got = run_k(F, w.XQ, w.WQ, w.x_scale, w.w_scale, offs)
    P.assert_rows_match(got.reshape(G * M, N), res, label=f"k_offsets cfg {cfg} seed {seed}")


@pytest.mark.parametrize("cfg", RAGGED_CONFIGS)
def test_n_offsets_equal_widths_bitwise_equal_batched(F, cfg):
    """Equal widths: column block g is the batched layout's slab g, bit for bit
    (same tile, same K order)."""
    rng = np.random.default_rng(301)
    G, M, Nw, K = 3, 70, 136, 336
    XQ, WQ = _codes(rng, (G, M, K)), _codes(rng, (G * Nw, K))
    xs, ws = _scales(rng, (G, M)), _scales(rng, G * Nw)
    with forced(cfg):
        a = run_n(F, XQ, WQ, xs, ws, [Nw, 2 * Nw, 3 * Nw])
        yb = F.f8f8bf16_rowwise_grouped_batched(P.dev(XQ), P.dev(WQ.reshape(G, Nw, K)), P.dev(xs),
                                                P.dev(ws.reshape(G, Nw)))
        torch.cuda.synchronize()
    b = P.bits_of(yb)
    for g in range(G):
        assert np.array_equal(a[:, g * Nw:(g + 1) * Nw], b[g])


@pytest.mark.parametrize("cfg", RAGGED_CONFIGS)
def test_k_offsets_concatenated_slabs_bitwise_equal_batched(F, cfg):
    """Slabs side by side along K: group g's output is the batched slab g, bit for bit."""
    rng = np.random.default_rng(302)
    G, M, N, K = 3, 45, 72, 208
    Xb, Wb = _codes(rng, (G, M, K)), _codes(rng, (G, N, K))
    xs, ws = _scales(rng, (G, M)), _scales(rng, (G, N))
    with forced(cfg):
        a = run_k(F, np.concatenate(list(Xb), axis=1), np.concatenate(list(Wb), axis=1), xs, ws,
                  [K, 2 * K, 3 * K])
        yb = F.f8f8bf16_rowwise_grouped_batched(P.dev(Xb), P.dev(Wb), P.dev(xs), P.dev(ws))
        torch.cuda.synchronize()
    assert np.array_equal(a, P.bits_of(yb))


def test_k_offsets_never_reads_past_its_slice(F):
    """Constant, single-signed data everywhere: each group's result is exactly its
    slice length, so a read past either end of the slice would show at once."""
    M, N, total_K = 40, 72, 1024
    XQ = np.full((M, total_K), 0x38, np.uint8)   # 1.0
    WQ = np.full((N, total_K), 0x38, np.uint8)
    lengths = [16, 0, 48, 400, 144, 16]
    offs = np.cumsum(lengths).tolist()
    ones_x, ones_w = np.ones((len(offs), M), np.float32), np.ones((len(offs), N), np.float32)
    for cfg in RAGGED_CONFIGS:
        with forced(cfg):
            got = oracle.bf16_bits_to_f64(run_k(F, XQ, WQ, ones_x, ones_w, offs))
        for g, n in enumerate(lengths):
            assert np.all(got[g] == n), f"cfg {cfg} group {g}: {np.unique(got[g])[:5]} != {n}"


def test_ragged_k_zero_zero_fills(F):
    rng = np.random.default_rng(303)
    got = run_n(F, np.zeros((2, 9, 0), np.uint8), np.zeros((16, 0), np.uint8), _scales(rng, (2, 9)),
                _scales(rng, 16), [8, 16])
    assert np.all(got == 0)
    got = run_k(F, np.zeros((9, 0), np.uint8), np.zeros((16, 0), np.uint8), _scales(rng, (2, 9)),
                _scales(rng, (2, 16)), [0, 0])
    assert np.all(got == 0)


def test_mm_rank_dispatch(F):
    """The grouped mm picks the layout from the operand ranks."""
    rng = np.random.default_rng(304)
    G, M, N, K = 2, 16, 32, 64
    XQ3, WQ2 = _codes(rng, (G, M, K)), _codes(rng, (G * N, K))
    xs, ws = _scales(rng, (G, M)), _scales(rng, G * N)
    offs = P.dev(np.array([N, 2 * N], np.int32))
    y = F.f8f8bf16_rowwise_grouped_mm(P.dev(XQ3), P.dev(WQ2), P.dev(xs), P.dev(ws), offs)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (M, G * N)
    assert np.array_equal(P.bits_of(y), run_n(F, XQ3, WQ2, xs, ws, [N, 2 * N]))
    with pytest.raises(ValueError, match="not accepted"):
        F.f8f8bf16_rowwise_grouped_mm_preshuffle(P.dev(XQ3), P.dev(WQ2), P.dev(xs), P.dev(ws), offs)


def test_full_size_n_offsets_workload(F):
    """The n_offsets bench workload at full size, checked on every column of 48
    sampled rows of each slab (the launch configuration the bench times)."""
    w = wl.moe_n_offsets()
    with forced(None):
        y = F.f8f8bf16_rowwise_grouped_n_offsets(P.dev(w.XQ), P.dev(w.WQ), P.dev(w.x_scale), P.dev(w.w_scale),
                                                 P.dev(w.n_offsets))
        torch.cuda.synchronize()
    got = P.bits_of(y)
    rows = np.sort(np.random.default_rng(305).choice(w.M, 48, replace=False))
    res = oracle.grouped_n_offsets(w.XQ[:, rows], w.WQ, w.x_scale[:, rows], w.w_scale, w.n_offsets)
    assert_cols_match(got[rows], res, "moe_n_offsets")


def test_full_size_k_offsets_workload(F):
    """The k_offsets bench workload at full size, checked on 32 sampled rows of
    every group's output."""
    w = wl.moe_wgrad_k_offsets()
    with forced(None):
        y = F.f8f8bf16_rowwise_grouped_k_offsets(P.dev(w.XQ), P.dev(w.WQ), P.dev(w.x_scale), P.dev(w.w_scale),
                                                 P.dev(w.k_offsets))
        torch.cuda.synchronize()
    got = P.bits_of(y)
    rows = np.sort(np.random.default_rng(306).choice(w.M, 32, replace=False))
    res = oracle.grouped_k_offsets(w.XQ[rows], w.WQ, w.x_scale[:, rows], w.w_scale, w.k_offsets)
    P.assert_rows_match(got[:, rows].reshape(-1, w.N), res, label="moe_wgrad_k_offsets")
