"""GPU parity for the block-scaled (groupwise) stacked GEMM.

Both kernel configurations are forced in turn on edge shapes (empty groups,
groups of 1 row, tile - 1 / tile + 1 rows, rows of no group, one and several
N and K blocks) and compared with the block-scaled oracle element by element;
the full-size workload is checked on sampled rows; shapes that are not whole
scale blocks are refused on the host.
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


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp8_rowwise_scaled_amd as F
    F.load()
    return F


@contextmanager
def forced(cfg):
    old = os.environ.get("FP8GG_BS_CONFIG")
    if cfg is None:
        os.environ.pop("FP8GG_BS_CONFIG", None)
    else:
        os.environ["FP8GG_BS_CONFIG"] = str(cfg)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("FP8GG_BS_CONFIG", None)
        else:
            os.environ["FP8GG_BS_CONFIG"] = old


def run(F, w, total_M):
    whole, y = P.guarded_output((total_M, w.N))
    F.f8f8bf16_groupwise_grouped_stacked(P.dev(w.XQ), P.dev(w.WQ), P.dev(w.x_scale), P.dev(w.w_scale),
                                         P.dev(w.M_sizes), out=y)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(y)


# (sizes, N, K, total_M): empty and 1-row groups, 127/129/257 rows, trailing rows of no group
CASES = [
    ([0, 3, 130, 257], 384, 640, None),
    ([1, 0, 127], 128, 128, 140),
    ([33, 31, 129], 256, 1152, None),
]


@pytest.mark.parametrize("cfg", [0, 1, 2])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_blockscale_matches_oracle(F, cfg, case):
    sizes, N, K, total_M = CASES[case]
    w = wl.make_stacked_blockscale(sizes, N, K, seed=900 + case, total_M=total_M)
    print(f"case blockscale cfg={cfg} sizes={sizes} N={N} K={K}", flush=True)
    with forced(cfg):
        got = run(F, w, w.total_M)
    res = oracle.grouped_stacked_blockscale(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
    P.assert_rows_match(got, res, label=f"blockscale cfg {cfg} case {case}")


def test_blockscale_refuses_partial_blocks_and_zero_fills_k_zero(F):
    w = wl.make_stacked_blockscale([4], 128, 128, seed=950)
    with pytest.raises(ValueError, match="multiples of 128"):
        F.f8f8bf16_groupwise_grouped_stacked(P.dev(w.XQ[:, :64].copy()), P.dev(w.WQ[:, :, :64].copy()),
                                             P.dev(w.x_scale), P.dev(w.w_scale), P.dev(w.M_sizes))
    from fp8_rowwise_scaled_amd import _lib
    a = 0x10000000
    st = _lib.load().f8f8bf16_groupwise_grouped_stacked(a, a, a, a, a, a + 0x1000000, 1, 4, 136, 128, None)
    assert st == _lib.ERR_UNSUPPORTED_SHAPE
    whole, y = P.guarded_output((3, 128))
    F.f8f8bf16_groupwise_grouped_stacked(torch.empty((3, 0), dtype=torch.uint8, device="cuda"),
                                         torch.empty((1, 128, 0), dtype=torch.uint8, device="cuda"),
                                         torch.empty((3, 0), dtype=torch.float32, device="cuda"),
                                         torch.empty((1, 1, 0), dtype=torch.float32, device="cuda"),
                                         P.dev(np.array([3], np.int64)), out=y)
    torch.cuda.synchronize()
    P.check_guards(whole)
    assert np.all(P.bits_of(y) == 0)


def test_full_size_blockscale_workload(F):
    """The block-scaled gate_up workload at full size (the configuration the bench
    times), checked on every column of 48 sampled rows."""
    w = wl.moe_gate_up_blockscale()
    with forced(None):
        got = run(F, w, w.total_M)
    rows = np.sort(np.random.default_rng(951).choice(w.total_M, 48, replace=False))
    owner = oracle.stacked_row_groups(w.M_sizes, w.total_M)[rows]
    for g in np.unique(owner):
        sel = rows[owner == g]
        sizes = np.zeros(w.G, np.int64)
        sizes[g] = sel.size
        res = oracle.grouped_stacked_blockscale(w.XQ[sel], w.WQ, w.x_scale[sel], w.w_scale, sizes)
        P.assert_rows_match(got[sel], res, rms=P.rms_of(res.bits), label=f"moe_gate_up_blockscale group {g}")


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_blockscale_preshuffled_weights_bitwise_equal_plain(F, cfg):
    """Pre-shuffled W through the same tile and K order: bit-identical to plain W."""
    w = wl.make_stacked_blockscale([0, 3, 130, 257], 384, 640, seed=960)
    WQs = F.f8f8bf16_shuffle_b(P.dev(w.WQ))
    with forced(cfg):
        plain = run(F, w, w.total_M)
        whole, y = P.guarded_output((w.total_M, w.N))
        F.f8f8bf16_groupwise_grouped_stacked_preshuffle(P.dev(w.XQ), WQs, P.dev(w.x_scale), P.dev(w.w_scale),
                                                        P.dev(w.M_sizes), out=y)
        torch.cuda.synchronize()
    P.check_guards(whole)
    assert np.array_equal(P.bits_of(y), plain)


@pytest.mark.parametrize("grid", [5, 7, 9])
def test_blockscale_persistent_grid_bitwise_equal_one_tile_schedule(F, grid):
    """The persistent schedule (config 2) on small grids: whole tiles plus quarter
    tiles (12 tiles on 5 workgroups), whole tiles only (7), two rounds of quarter
    tiles after the whole ones (9; the default grid of 256 runs only quarters):
    each output element is computed by one workgroup in the same K
    order, so the result equals the one-tile-per-workgroup schedule (config 0)
    bit for bit, and the oracle within the tolerance."""
    w = wl.make_stacked_blockscale([0, 3, 130, 257], 384, 640, seed=970)
    with forced(0):
        ref = run(F, w, w.total_M)
    old = os.environ.get("FP8GG_TAIL_GRID")
    os.environ["FP8GG_TAIL_GRID"] = str(grid)
    try:
        with forced(2):
            got = run(F, w, w.total_M)
    finally:
        if old is None:
            os.environ.pop("FP8GG_TAIL_GRID", None)
        else:
            os.environ["FP8GG_TAIL_GRID"] = old
    assert np.array_equal(got, ref)
    res = oracle.grouped_stacked_blockscale(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
    P.assert_rows_match(got, res, label=f"blockscale persistent grid {grid}")


def test_blockscale_long_k(F):
    """K = 28672 (224 scale blocks, the dense-expert depth): 224 scaled partial sums
    per output; both the persistent and the one-tile schedules against the oracle
    on every column of sampled rows."""
    w = wl.make_stacked_blockscale([300, 0, 212], 512, 28672, seed=980)
    rows = np.sort(np.random.default_rng(981).choice(w.total_M, 24, replace=False))
    owner = oracle.stacked_row_groups(w.M_sizes, w.total_M)[rows]
    for cfg in (2, 0):
        with forced(cfg):
            got = run(F, w, w.total_M)
        for g in np.unique(owner):
            sel = rows[owner == g]
            sizes = np.zeros(w.G, np.int64)
            sizes[g] = sel.size
            res = oracle.grouped_stacked_blockscale(w.XQ[sel], w.WQ, w.x_scale[sel], w.w_scale, sizes)
            P.assert_rows_match(got[sel], res, rms=P.rms_of(res.bits), label=f"long K cfg {cfg} group {g}")


def _dynamic_inputs(zsi, em, N, K, seed):
    """Padded-layout block-scaled inputs: every slab row drawn and quantised per
    (row, 128) block, W per 128 x 128 block (the stacked generator, reshaped)."""
    G = len(zsi)
    w = wl.make_stacked_blockscale([em] * G, N, K, seed=seed)
    return (w.XQ.reshape(G, em, K), w.WQ, w.x_scale.reshape(G, em, K // 128), w.w_scale,
            np.asarray(zsi, np.int64))


def run_dynamic(F, XQ, WQ, xs, ws, zsi, zeroing, pre=False):
    G, em, _ = XQ.shape
    whole, y = P.guarded_output((G, em, WQ.shape[1]))
    fn = F.f8f8bf16_groupwise_grouped_dynamic_preshuffle if pre else F.f8f8bf16_groupwise_grouped_dynamic
    Wd = F.f8f8bf16_shuffle_b(P.dev(WQ)) if pre else P.dev(WQ)
    fn(P.dev(XQ), Wd, P.dev(xs), P.dev(ws), P.dev(zsi), zeroing_output_tensor=zeroing, out=y)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(y)


@pytest.mark.parametrize("cfg", [0, 1])
@pytest.mark.parametrize("zeroing", [True, False])
def test_dynamic_blockscale_matches_oracle(F, cfg, zeroing):
    """Slabs of 200 rows (the last M tile overhangs the slab), valid counts 0, full,
    37, past the slab (clamped) and 129, padding zeroed or left untouched."""
    XQ, WQ, xs, ws, zsi = _dynamic_inputs([0, 200, 37, 205, 129], 200, 256, 384, seed=990)
    with forced(cfg):
        got = run_dynamic(F, XQ, WQ, xs, ws, zsi, zeroing)
    res = oracle.grouped_dynamic_blockscale(XQ, WQ, xs, ws, zsi, zeroing)
    P.assert_rows_match(got.reshape(-1, WQ.shape[1]), res, label=f"dynamic blockscale cfg {cfg} zeroing {zeroing}")


@pytest.mark.parametrize("cfg", [0, 1])
def test_dynamic_blockscale_bitwise_equal_stacked_on_compacted_rows_and_preshuffled(F, cfg):
    XQ, WQ, xs, ws, zsi = _dynamic_inputs([3, 0, 130, 64], 160, 384, 512, seed=991)
    G, em, K = XQ.shape
    with forced(cfg):
        d = run_dynamic(F, XQ, WQ, xs, ws, zsi, True)
        dp = run_dynamic(F, XQ, WQ, xs, ws, zsi, True, pre=True)
        rows = np.concatenate([g * em + np.arange(zsi[g]) for g in range(G)]).astype(np.int64)
        y = F.f8f8bf16_groupwise_grouped_stacked(P.dev(XQ.reshape(G * em, K)[rows]), P.dev(WQ),
                                                 P.dev(xs.reshape(G * em, -1)[rows]), P.dev(ws), P.dev(zsi))
        torch.cuda.synchronize()
    assert np.array_equal(dp, d)
    assert np.array_equal(d.reshape(G * em, -1)[rows], P.bits_of(y))


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_offsets_and_batched_blockscale_bitwise_equal_stacked(F, cfg):
    """The offsets layout (int32 prefix of the same row counts) and the batched
    layout (equal slabs) run the stacked layout's tiles and K order: bit-identical
    results on the same rows, for every configuration; and the oracle within the
    tolerance."""
    w = wl.make_stacked_blockscale([0, 3, 130, 257], 384, 640, seed=995)
    offs = P.dev(np.cumsum(w.M_sizes).astype(np.int32))
    with forced(cfg):
        st = run(F, w, w.total_M)
        whole, y = P.guarded_output((w.total_M, w.N))
        F.f8f8bf16_groupwise_grouped_offsets(P.dev(w.XQ), P.dev(w.WQ), P.dev(w.x_scale), P.dev(w.w_scale), offs,
                                             out=y)
        torch.cuda.synchronize()
        P.check_guards(whole)
        of = P.bits_of(y)
    assert np.array_equal(of, st)
    res = oracle.grouped_offsets_blockscale(w.XQ, w.WQ, w.x_scale, w.w_scale, np.cumsum(w.M_sizes).astype(np.int32))
    P.assert_rows_match(of, res, label=f"offsets blockscale cfg {cfg}")

    G, M = 3, 150
    b = wl.make_stacked_blockscale([M] * G, 256, 512, seed=996)
    with forced(cfg):
        st = run(F, b, b.total_M)
        whole, y = P.guarded_output((G, M, b.N))
        F.f8f8bf16_groupwise_grouped_batched(P.dev(b.XQ.reshape(G, M, -1)), P.dev(b.WQ),
                                             P.dev(b.x_scale.reshape(G, M, -1)), P.dev(b.w_scale), out=y)
        torch.cuda.synchronize()
        P.check_guards(whole)
        ba = P.bits_of(y)
    assert np.array_equal(ba.reshape(G * M, -1), st)
    res = oracle.grouped_batched_blockscale(b.XQ.reshape(G, M, -1), b.WQ, b.x_scale.reshape(G, M, -1), b.w_scale)
    P.assert_rows_match(ba.reshape(G * M, -1), res, label=f"batched blockscale cfg {cfg}")


@pytest.mark.parametrize("cfg", [2, 3])
def test_blockscale_forced_config_refusals(F, cfg):
    """The persistent configuration (2) walks packed rows only, so the padded
    layout refuses it before any launch; configuration 3 does not exist."""
    XQ, WQ, xs, ws, zsi = _dynamic_inputs([3, 5], 64, 128, 256, seed=995)
    with forced(cfg):
        with pytest.raises(ValueError, match="not a configuration"):
            run_dynamic(F, XQ, WQ, xs, ws, zsi, True)
