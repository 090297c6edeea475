"""GPU tests of the persistent schedule (stacked layout).

Configurations 16 and 17 (and 26 on pre-shuffled weights) run one workgroup per
compute unit over the output tiles in data-parallel order.  When the tile count T
is not a multiple of the grid, the tiles of the last round may run as quarter
tiles.  FP8GG_TAIL forces the remainder mode (1 whole tiles, 2 quarter tiles) and
FP8GG_TAIL_GRID the grid.  Every output element is computed by one workgroup in
the K order of the data-parallel kernel, so besides matching the oracle the
output must equal the data-parallel twin's bit for bit in every mode and grid.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests import parity as P

pytestmark = pytest.mark.gpu

PERSISTENT = {16: (256, 256, 7), 17: (128, 256, 9)}   # id -> (BM, BN, data-parallel twin)
ENV = ("FP8GG_CONFIG", "FP8GG_TAIL", "FP8GG_TAIL_GRID")


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

    def set_env(**kw):
        for k, v in kw.items():
            name = "FP8GG_" + k.upper()
            if v is None:
                os.environ.pop(name, None)
            else:
                os.environ[name] = str(v)
    yield set_env
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def tail_shape(BM, BN, extra_tiles):
    """Three groups (one empty), ragged sizes, 16 N tiles: T = 16 * m_tiles tiles
    with T >= cus() + extra_tiles, so the last round is partial.  The last group's
    final M tile holds fewer than BM / 2 rows, so two of its quarters are empty."""
    m_tiles = -(-(cus() + extra_tiles) // 16)
    a = m_tiles // 2
    return [BM * a - 3, 0, BM * (m_tiles - a - 1) + BM // 2 - 5], 16 * BN


_cache = {}


def case(sizes, N, K, seed):
    key = (tuple(sizes), N, K, seed)
    if key not in _cache:
        w = wl.make_stacked(sizes, N, K, seed=seed)
        ref = oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
        _cache.clear()
        _cache[key] = (w, ref)
    return _cache[key]


def run(F, w, stream=None, pre=False):
    whole, out = P.guarded_output((w.total_M, w.N))
    args = [P.dev(a) for a in (w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)]
    fn = F.f8f8bf16_rowwise_grouped_stacked
    if pre:
        args[1] = F.f8f8bf16_shuffle_b(args[1])
        fn = F.f8f8bf16_rowwise_grouped_stacked_preshuffle
    if stream is None:
        fn(*args, out=out)
    else:
        with torch.cuda.stream(stream):
            fn(*args, out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(out)


@pytest.mark.parametrize("cfg", sorted(PERSISTENT))
@pytest.mark.parametrize("K", [2048, 2064])
@pytest.mark.parametrize("tail", [None, 1, 2])
def test_persistent_matches_oracle_and_data_parallel(F, env, cfg, K, tail):
    BM, BN, twin = PERSISTENT[cfg]
    sizes, N = tail_shape(BM, BN, extra_tiles=37)
    w, ref = case(sizes, N, K, seed=1400 + cfg)
    print(f"case persistent cfg={cfg} sizes={sizes} N={N} K={K} tail={tail} cus={cus()}", flush=True)
    env(config=cfg, tail=tail)
    got = run(F, w)
    P.assert_rows_match(got, ref, label=f"persistent cfg{cfg} K={K} tail={tail}")
    env(config=twin, tail=None)
    assert np.array_equal(run(F, w), got)


@pytest.mark.parametrize("K", [2048, 1040])
@pytest.mark.parametrize("tail", [None, 1, 2])
def test_fewer_tiles_than_workgroups(F, env, K, tail):
    """T < grid: every tile is in the last round (quarters when asked or chosen)."""
    sizes = [300, 0, 77]                      # 3 + 1 M tiles of 128 rows
    w = wl.make_stacked(sizes, 1024, K, seed=1800 + K)
    print(f"case small sizes={sizes} K={K} tail={tail}", flush=True)
    env(config=17, tail=tail)
    got = run(F, w)
    ref = oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
    P.assert_rows_match(got, ref, label=f"few tiles K={K} tail={tail}")
    env(config=9, tail=None)
    assert np.array_equal(run(F, w), got)


@pytest.mark.parametrize("grid", [37, 100])
@pytest.mark.parametrize("tail", [None, 2])
def test_other_grid_sizes(F, env, grid, tail):
    BM, BN, twin = PERSISTENT[17]
    sizes, N = tail_shape(BM, BN, extra_tiles=5)
    w, ref = case(sizes, N, 2064, seed=1417)
    print(f"case grid={grid} tail={tail} sizes={sizes}", flush=True)
    env(config=17, tail_grid=grid, tail=tail)
    got = run(F, w)
    P.assert_rows_match(got, ref, label=f"grid {grid} tail {tail}")
    env(config=twin, tail_grid=None, tail=None)
    assert np.array_equal(run(F, w), got)


def test_n_not_a_multiple_of_the_tile(F, env):
    """N = 16 * 256 - 136: the last N tile's right quarters lie past N."""
    sizes = [700, 0, 301]
    N = 16 * 256 - 136
    w = wl.make_stacked(sizes, N, 1024, seed=1901)
    ref = oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
    print(f"case ntail sizes={sizes} N={N}", flush=True)
    env(config=16, tail=2)
    got = run(F, w)
    P.assert_rows_match(got, ref, label="quarters with an N tail")
    env(config=7, tail=None)
    assert np.array_equal(run(F, w), got)


@pytest.mark.parametrize("tail", [None, 1, 2])
def test_preshuffled_persistent_kernel(F, env, tail):
    """Configuration 26 (pre-shuffled weights) against the oracle and bitwise
    against its data-parallel twin 25."""
    sizes, N = tail_shape(256, 256, extra_tiles=37)
    w, ref = case(sizes, N, 2048, seed=1426)
    print(f"case preshuffled persistent sizes={sizes} tail={tail}", flush=True)
    env(config=26, tail=tail)
    got = run(F, w, pre=True)
    P.assert_rows_match(got, ref, label=f"preshuffled persistent tail={tail}")
    env(config=25, tail=None)
    assert np.array_equal(run(F, w, pre=True), got)


def test_persistent_on_a_second_stream(F, env):
    BM, BN, _ = PERSISTENT[17]
    sizes, N = tail_shape(BM, BN, extra_tiles=5)
    w, _ = case(sizes, N, 2064, seed=1417)
    env(config=17, tail=2)
    a = run(F, w)
    s = torch.cuda.Stream()
    b = run(F, w, stream=s)
    assert np.array_equal(a, b)


def test_persistent_under_graph_capture(F, env):
    """The persistent kernel itself is captured (it uses no library memory); every
    replay matches the oracle and the eager result bitwise."""
    BM, BN, _ = PERSISTENT[16]
    sizes, N = tail_shape(BM, BN, extra_tiles=11)
    w, ref = case(sizes, N, 1024, seed=1700)
    args = [P.dev(a) for a in (w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)]
    env(config=16, tail=None)
    expect = run(F, w)
    out = torch.empty((w.total_M, N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        F.f8f8bf16_rowwise_grouped_stacked(*args, out=out)
    for rep in range(3):
        out.view(torch.int16).fill_(P.SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = P.bits_of(out)
        P.assert_rows_match(got, ref, label=f"graph replay {rep}")
        assert np.array_equal(got, expect)


def test_gate_up_default_plan_is_persistent(F):
    p = F.plan(F.LAYOUT_STACKED, False, 8, 4096, 4096, 7168)
    assert p["persistent"] == 1
