"""GPU tests of the persistent schedule with a split last wave (stacked layout).

Configurations 16 and 17 run one workgroup per compute unit over the output tiles
in data-parallel order and cut the tiles of the last, partial wave along K into
pieces whose fp32 partial sums are combined through a workspace.  Shapes here give
a tile count T that is not a multiple of the grid, so the tail is split; the
split factor is left to the library or forced with FP8GG_TAIL_SPLIT, and the grid
with FP8GG_TAIL_GRID.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests import parity as P

pytestmark = pytest.mark.gpu

TAIL_CONFIGS = {16: (256, 256, 7), 17: (128, 256, 9)}   # id -> (BM, BN, data-parallel twin)
ENV = ("FP8GG_CONFIG", "FP8GG_TAIL_SPLIT", "FP8GG_TAIL_GRID")


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
    with T >= cus() + extra_tiles, so the last wave is partial."""
    m_tiles = -(-(cus() + extra_tiles) // 16)
    a = m_tiles // 2
    return [BM * a - 3, 0, BM * (m_tiles - a) - 1], 16 * BN


def tile_rows(sizes, BM):
    """Row ranges [r0, r1) of the M tiles, in tile order."""
    out, start = [], 0
    for s in sizes:
        for j in range(-(-s // BM)):
            out.append((start + j * BM, min(start + (j + 1) * BM, start + s)))
        start += s
    return out


def split_mask(sizes, BM, BN, N, grid):
    """Boolean [rows, N] mask of the outputs in the last-wave tiles (those that may be
    split when the split factor is above one)."""
    rows = tile_rows(sizes, BM)
    n_tiles = N // BN
    T = len(rows) * n_tiles
    rem = T % grid
    mask = np.zeros((sum(sizes), N), dtype=bool)
    for tile in range(T - rem, T):
        r0, r1 = rows[tile // n_tiles]
        c0 = (tile % n_tiles) * BN
        mask[r0:r1, c0:c0 + BN] = True
    return mask, T, rem


_cache = {}


def case(sizes, N, K, seed):
    key = (tuple(sizes), N, K, seed)
    if key not in _cache:
        w = wl.make_stacked(sizes, N, K, seed=seed)
        ref = oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
        _cache.clear()
        _cache[key] = (w, ref)
    return _cache[key]


def run(F, w, stream=None):
    whole, out = P.guarded_output((w.total_M, w.N))
    args = [P.dev(a) for a in (w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)]
    if stream is None:
        F.f8f8bf16_rowwise_grouped_stacked(*args, out=out)
    else:
        with torch.cuda.stream(stream):
            F.f8f8bf16_rowwise_grouped_stacked(*args, out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(out)


@pytest.mark.parametrize("cfg", sorted(TAIL_CONFIGS))
@pytest.mark.parametrize("K", [2048, 2064])
@pytest.mark.parametrize("split", [None, 2, 16])
def test_split_tail_matches_oracle(F, env, cfg, K, split):
    BM, BN, _ = TAIL_CONFIGS[cfg]
    sizes, N = tail_shape(BM, BN, extra_tiles=37)
    w, ref = case(sizes, N, K, seed=1400 + cfg)
    print(f"case split-tail cfg={cfg} sizes={sizes} N={N} K={K} split={split} cus={cus()}", flush=True)
    env(config=cfg, tail_split=split)
    got = run(F, w)
    P.assert_rows_match(got, ref, label=f"split tail cfg{cfg} K={K} split={split}")
    # repeated calls give the same bits: counters were reset, partials added in piece order
    assert np.array_equal(run(F, w), got)


@pytest.mark.parametrize("cfg", sorted(TAIL_CONFIGS))
def test_unsplit_persistent_equals_data_parallel(F, env, cfg):
    """With the split forced off, the persistent kernel computes every tile exactly
    as the data-parallel kernel does: bitwise equal outputs."""
    BM, BN, twin = TAIL_CONFIGS[cfg]
    sizes, N = tail_shape(BM, BN, extra_tiles=37)
    w, _ = case(sizes, N, 2064, seed=1400 + cfg)
    print(f"case unsplit cfg={cfg} sizes={sizes}", flush=True)
    env(config=cfg, tail_split=1)
    persistent = run(F, w)
    env(config=twin, tail_split=None)
    dp = run(F, w)
    assert np.array_equal(persistent, dp)


@pytest.mark.parametrize("cfg", sorted(TAIL_CONFIGS))
def test_only_last_wave_tiles_differ_from_data_parallel(F, env, cfg):
    BM, BN, twin = TAIL_CONFIGS[cfg]
    sizes, N = tail_shape(BM, BN, extra_tiles=37)
    w, ref = case(sizes, N, 2048, seed=1400 + cfg)
    env(config=cfg, tail_split=4)
    split = run(F, w)
    env(config=twin, tail_split=None)
    dp = run(F, w)
    mask, T, rem = split_mask(sizes, BM, BN, N, cus())
    print(f"case last-wave cfg={cfg} T={T} rem={rem}", flush=True)
    assert 0 < rem < T
    assert np.array_equal(split[~mask], dp[~mask])
    P.assert_rows_match(split, ref, label="split tail")


@pytest.mark.parametrize("K", [2048, 1040])
@pytest.mark.parametrize("split", [None, 4])
def test_fewer_tiles_than_workgroups(F, env, K, split):
    """T < grid: every tile is in the last wave (and is split when asked to)."""
    sizes = [300, 0, 77]                      # 3 + 1 M tiles of 128 rows
    w = wl.make_stacked(sizes, 1024, K, seed=1800 + K)
    print(f"case small sizes={sizes} K={K} split={split}", flush=True)
    env(config=17, tail_split=split)
    got = run(F, w)
    ref = oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
    P.assert_rows_match(got, ref, label=f"all tiles split K={K}")
    assert np.array_equal(run(F, w), got)


@pytest.mark.parametrize("grid", [37, 100])
def test_other_grid_sizes(F, env, grid):
    BM, BN, _ = TAIL_CONFIGS[17]
    sizes, N = tail_shape(BM, BN, extra_tiles=5)
    w, ref = case(sizes, N, 2064, seed=1417)
    print(f"case grid={grid} sizes={sizes}", flush=True)
    env(config=17, tail_grid=grid, tail_split=None)
    got = run(F, w)
    P.assert_rows_match(got, ref, label=f"grid {grid}")


@pytest.mark.parametrize("split", [None, 3])
def test_preshuffled_persistent_kernel(F, env, split):
    """The persistent kernel on pre-shuffled weights (configuration 26), whole and
    split tiles, against the oracle and bitwise against its data-parallel twin when
    unsplit."""
    sizes, N = tail_shape(256, 256, extra_tiles=37)
    w, ref = case(sizes, N, 2048, seed=1426)
    print(f"case preshuffled persistent sizes={sizes} split={split}", flush=True)
    args = [P.dev(a) for a in (w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)]
    args[1] = F.f8f8bf16_shuffle_b(args[1])

    def run_pre():
        whole, out = P.guarded_output((w.total_M, w.N))
        F.f8f8bf16_rowwise_grouped_stacked_preshuffle(*args, out=out)
        torch.cuda.synchronize()
        P.check_guards(whole)
        return P.bits_of(out)

    env(config=26, tail_split=split)
    got = run_pre()
    P.assert_rows_match(got, ref, label=f"preshuffled persistent split={split}")
    assert np.array_equal(run_pre(), got)
    if split is None:
        env(config=26, tail_split=1)
        unsplit = run_pre()
        env(config=25, tail_split=None)
        assert np.array_equal(unsplit, run_pre())


def test_split_tail_on_a_second_stream(F, env):
    BM, BN, _ = TAIL_CONFIGS[17]
    sizes, N = tail_shape(BM, BN, extra_tiles=5)
    w, _ = case(sizes, N, 2064, seed=1417)
    env(config=17, tail_split=None)
    a = run(F, w)
    s = torch.cuda.Stream()
    b = run(F, w, stream=s)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("warm", [False, True])
def test_split_tail_under_graph_capture(F, env, warm):
    """A captured call runs the data-parallel twin, whether or not the capturing
    stream already has a workspace (warm: an eager call on it first); replays match
    the oracle every time and the twin bitwise."""
    BM, BN, twin = TAIL_CONFIGS[16]
    sizes, N = tail_shape(BM, BN, extra_tiles=11)
    w, ref = case(sizes, N, 1024, seed=1700)
    args = [P.dev(a) for a in (w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)]
    env(config=twin, tail_split=None)
    expect = run(F, w)
    env(config=16, tail_split=None)
    out = torch.empty((w.total_M, N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.Stream()
    if warm:
        with torch.cuda.stream(stream):
            F.f8f8bf16_rowwise_grouped_stacked(*args, out=out)
        torch.cuda.synchronize()
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


def test_gate_up_default_plan_is_split_tail(F):
    p = F.plan(F.LAYOUT_STACKED, False, 8, 4096, 4096, 7168)
    assert p["split_tail"] == 1
