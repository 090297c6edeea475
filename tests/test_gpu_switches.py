"""GPU tests of the two scheduling switches that only reorder or skip work.

* FP8GG_XCD: the padded layout's data-parallel grid (rowwise and block-scaled) and
  the n_offsets grid hand each XCD a contiguous share of their tiles (the default)
  instead of every eighth tile.  Every tile is still computed by one workgroup in
  the same K order.
* FP8GG_SKIP_DEAD: a wave whose rows all lie past its tile's group reads no
  fragments and issues no MFMAs (the default); those outputs are never stored.

Neither may change a single output bit: each case is checked against the oracle
and bitwise against the same call with the switch off.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests import parity as P

pytestmark = pytest.mark.gpu

ENV = ("FP8GG_XCD", "FP8GG_SKIP_DEAD", "FP8GG_CONFIG", "FP8GG_TAIL_GRID")


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp8_rowwise_scaled_amd as F
    F.load()
    return F


@pytest.fixture
def env():
    saved = {k: os.environ.get(k) for k in ENV}

    def set_env(name, value):
        if value is None:
            os.environ.pop(name, None)
        else:
            os.environ[name] = str(value)
    yield set_env
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


def run_padded(F, w, zeroing):
    whole, out = P.guarded_output((w.G, w.expected_m, w.N))
    args = [P.dev(a) for a in (w.XQ, w.WQ, w.x_scale, w.w_scale, w.zero_start_index_M)]
    F.f8f8bf16_rowwise_grouped_dynamic(*args, zeroing_output_tensor=zeroing, out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(out)


def run_stacked(F, w, pre=False):
    whole, out = P.guarded_output((w.total_M, w.N))
    args = [P.dev(a) for a in (w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)]
    fn = F.f8f8bf16_rowwise_grouped_stacked
    if pre:
        args[1] = F.f8f8bf16_shuffle_b(args[1])
        fn = F.f8f8bf16_rowwise_grouped_stacked_preshuffle
    fn(*args, out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(out)


@pytest.mark.parametrize("zeroing", [True, False])
@pytest.mark.parametrize("K", [1024, 1040])
def test_padded_xcd_order_is_bitwise_neutral(F, env, zeroing, K):
    """16 slabs of 512 rows (128x256 tiles, grid 16 x 4 x 4 = 256 workgroups, a
    multiple of 8): empty, full and ragged slabs, N = 1000 (an N tail)."""
    zsi = np.array([0, 512, 141, 272, 339, 132, 218, 294, 393, 466, 259, 272, 455, 300, 169, 61], np.int64)
    w = wl.make_dynamic(zsi, 512, 1000, K, seed=7700 + K)
    ref = oracle.grouped_dynamic(w.XQ, w.WQ, w.x_scale, w.w_scale, w.zero_start_index_M, zeroing)
    print(f"case padded xcd K={K} zeroing={zeroing}", flush=True)
    env("FP8GG_XCD", None)
    got = run_padded(F, w, zeroing)
    P.assert_rows_match(got.reshape(-1, w.N), ref, label=f"padded xcd order K={K}")
    env("FP8GG_XCD", 0)
    assert np.array_equal(run_padded(F, w, zeroing), got)


@pytest.mark.parametrize("G,M,cfg", [(8, 512, None), (5, 300, 9), (12, 40, 18), (3, 64, 2)])
def test_n_offsets_xcd_order_is_bitwise_neutral(F, env, G, M, cfg):
    """The n_offsets grid in XCD order (its default), on grids that are and are not
    multiples of 8: ragged column groups (one empty, one of 8 columns), an N tail."""
    from tests.test_gpu_ragged import assert_cols_match
    rng = np.random.default_rng(7900 + G)
    widths = 8 * rng.integers(1, 60, G)
    widths[0] = 0
    widths[-1] = 8
    w = wl.make_n_offsets(widths, M, 384, seed=7900 + G, total_N=int(widths.sum()) + 16)
    offs = np.cumsum(widths).astype(np.int32)
    ref = oracle.grouped_n_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, offs)
    args = [P.dev(a) for a in (w.XQ, w.WQ, w.x_scale, w.w_scale)] + [P.dev(offs)]

    def run():
        whole, y = P.guarded_output((M, w.WQ.shape[0]))
        F.f8f8bf16_rowwise_grouped_n_offsets(*args, out=y)
        torch.cuda.synchronize()
        P.check_guards(whole)
        return P.bits_of(y)

    print(f"case n_offsets xcd G={G} M={M} cfg={cfg}", flush=True)
    env("FP8GG_CONFIG", cfg)
    env("FP8GG_XCD", None)
    got = run()
    assert_cols_match(got, ref, f"n_offsets xcd order G={G}")
    env("FP8GG_XCD", 0)
    assert np.array_equal(run(), got)


@pytest.mark.parametrize("zeroing", [True, False])
@pytest.mark.parametrize("pre", [False, True])
def test_padded_blockscale_xcd_order_is_bitwise_neutral(F, env, zeroing, pre):
    """The block-scaled padded grid in XCD order (its default for 128x256 tiles):
    16 slabs of 512 rows, N = 1024, K = 1024 (whole 128-wide blocks)."""
    zsi = np.array([0, 512, 141, 272, 339, 132, 218, 294, 393, 466, 259, 272, 455, 300, 169, 61], np.int64)
    d = wl.make_dynamic_blockscale(zsi, 512, 1024, 1024, seed=7800)
    ref = oracle.grouped_dynamic_blockscale(d.XQ, d.WQ, d.x_scale, d.w_scale, d.zero_start_index_M, zeroing)
    args = [P.dev(a) for a in (d.XQ, d.WQ, d.x_scale, d.w_scale, d.zero_start_index_M)]
    fn = F.f8f8bf16_groupwise_grouped_dynamic
    if pre:
        args[1] = F.f8f8bf16_shuffle_b(args[1])
        fn = F.f8f8bf16_groupwise_grouped_dynamic_preshuffle

    def run():
        whole, out = P.guarded_output((d.G, d.expected_m, d.N))
        fn(*args, zeroing_output_tensor=zeroing, out=out)
        torch.cuda.synchronize()
        P.check_guards(whole)
        return P.bits_of(out)

    print(f"case padded blockscale xcd pre={pre} zeroing={zeroing}", flush=True)
    env("FP8GG_XCD", None)
    got = run()
    P.assert_rows_match(got.reshape(-1, d.N), ref, label=f"padded blockscale xcd order pre={pre}")
    env("FP8GG_XCD", 0)
    assert np.array_equal(run(), got)


# (pre-shuffled W, forced configuration, persistent grid): the default plan is the
# persistent 256x256 kernel; its 18 tiles make quarter tiles on the full grid and
# whole tiles on a grid of 5; the rest are data-parallel tiles.
DEAD_CASES = [(False, None, None), (False, None, 5), (False, 0, None), (False, 7, None), (False, 9, None),
              (True, None, None), (True, None, 5), (True, 25, None), (True, 4, None)]


@pytest.mark.parametrize("pre,cfg,grid", DEAD_CASES)
def test_dead_waves_are_bitwise_neutral(F, env, pre, cfg, grid):
    """Groups whose last M tile holds a few rows (20, 27, 84 rows past a multiple of
    256): the waves of those tiles that hold no row skip their MFMAs."""
    sizes = [256 * 3 + 20, 0, 256 + 84, 27, 256 * 2]
    w = wl.make_stacked(sizes, 512, 1024, seed=7800)
    ref = oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
    print(f"case dead waves pre={pre} cfg={cfg} grid={grid}", flush=True)
    env("FP8GG_CONFIG", cfg)
    env("FP8GG_TAIL_GRID", grid)
    env("FP8GG_SKIP_DEAD", None)
    got = run_stacked(F, w, pre)
    P.assert_rows_match(got, ref, label=f"dead waves pre={pre} cfg={cfg} grid={grid}")
    env("FP8GG_SKIP_DEAD", 0)
    assert np.array_equal(run_stacked(F, w, pre), got)
