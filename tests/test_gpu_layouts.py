"""GPU parity for the offsets (int32 inclusive prefix) and batched (3D-3D) layouts.

Every kernel configuration is forced in turn on edge shapes (group sizes 0, 1,
tile - 1, tile, tile + 1; N and K tails) and compared with the oracle element by
element; offsets are also compared bitwise with the stacked entry point on the
same rows, and the batched layout with the stacked one on the flattened slabs.
The persistent configurations are run on shapes whose last round runs as quarter
tiles.
"""
import os

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


def _configs(layout: int, preshuffled: bool):
    """Configuration ids the host planner accepts for a layout (forced in turn)."""
    import fp8_rowwise_scaled_amd as F
    from fp8_rowwise_scaled_amd import _lib
    ids = []
    old = os.environ.get("FP8GG_CONFIG")
    try:
        for c in range(_lib.load().f8f8bf16_num_configs()):
            os.environ["FP8GG_CONFIG"] = str(c)
            try:
                F.plan(layout, preshuffled, 2, 64, 64, 128)
                ids.append(c)
            except ValueError:
                pass
    finally:
        if old is None:
            os.environ.pop("FP8GG_CONFIG", None)
        else:
            os.environ["FP8GG_CONFIG"] = old
    return ids


from fp8_rowwise_scaled_amd import _lib as _L  # noqa: E402

PLAIN = _configs(_L.LAYOUT_OFFSETS, False)
PRE = _configs(_L.LAYOUT_OFFSETS, True)


@pytest.fixture
def config_env():
    keys = ("FP8GG_CONFIG", "FP8GG_TAIL")
    saved = {k: os.environ.get(k) for k in keys}

    def set_cfg(c, tail=None):
        for k, v in (("FP8GG_CONFIG", c), ("FP8GG_TAIL", tail)):
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = str(v)
    yield set_cfg
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


def run_offsets(F, w, offsets, pre=False):
    whole, out = P.guarded_output((w.total_M, w.N))
    W = P.dev(w.WQ)
    fn = F.f8f8bf16_rowwise_grouped_offsets
    if pre:
        W = F.f8f8bf16_shuffle_b(W)
        fn = F.f8f8bf16_rowwise_grouped_offsets_preshuffle
    fn(P.dev(w.XQ), W, P.dev(w.x_scale), P.dev(w.w_scale),
       torch.from_numpy(np.asarray(offsets, np.int32)).cuda(), out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(out)


def run_stacked(F, w, pre=False):
    whole, out = P.guarded_output((w.total_M, w.N))
    W = P.dev(w.WQ)
    fn = F.f8f8bf16_rowwise_grouped_stacked
    if pre:
        W = F.f8f8bf16_shuffle_b(W)
        fn = F.f8f8bf16_rowwise_grouped_stacked_preshuffle
    fn(P.dev(w.XQ), W, P.dev(w.x_scale), P.dev(w.w_scale), P.dev(w.M_sizes), out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(out)


def run_batched(F, d, pre=False):
    G, M, _ = d.XQ.shape
    whole, out = P.guarded_output((G, M, d.N))
    W = P.dev(d.WQ)
    fn = F.f8f8bf16_rowwise_grouped_batched
    if pre:
        W = F.f8f8bf16_shuffle_b(W)
        fn = F.f8f8bf16_rowwise_grouped_batched_preshuffle
    fn(P.dev(d.XQ), W, P.dev(d.x_scale), P.dev(d.w_scale), out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(out)


def batched_case(G, M, N, K, seed):
    return wl.make_dynamic([M] * G, M, N, K, seed=seed)


# ---------------------------------------------------------------------------
# offsets
# ---------------------------------------------------------------------------

OFFSETS_EDGES = [
    # (offsets, N, K, total_M)
    ([0, 1, 32, 64, 97], 136, 16, 97),
    ([63, 127, 192, 192], 264, 112, 192),
    ([127, 255, 384], 56, 144, 384),
    ([255, 255, 511, 768], 1000, 320, 768),
    ([3, 3, 3, 8], 8, 208, 20),             # rows 8.. belong to no group
    ([50, 20, 90, 400], 264, 64, 120),      # a decreasing offset (empty group); past total_M
    ([-5, 40], 56, 128, 40),                # a negative offset (empty group)
]


def _offsets_problem(case, seed):
    offsets, N, K, total_M = OFFSETS_EDGES[case]
    w = wl.make_stacked([total_M] + [0] * (len(offsets) - 1), N, K, seed=seed)
    return w, np.asarray(offsets, np.int32)


@pytest.mark.parametrize("cfg", PLAIN)
@pytest.mark.parametrize("case", range(len(OFFSETS_EDGES)))
def test_offsets_edges_every_config(F, config_env, cfg, case):
    w, offs = _offsets_problem(case, 500 + case)
    config_env(cfg)
    print(f"case offsets cfg={cfg} offsets={offs.tolist()} N={w.N} K={w.K} total_M={w.total_M}", flush=True)
    ref = oracle.grouped_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, offs)
    got = run_offsets(F, w, offs)
    P.assert_rows_match(got, ref, label=f"offsets cfg{cfg}/case{case}")
    if np.all(np.diff(np.concatenate([[0], offs])) >= 0) and offs[-1] <= w.total_M:
        w.M_sizes = np.diff(np.concatenate([[0], offs])).astype(np.int64)
        assert np.array_equal(run_stacked(F, w), got)


@pytest.mark.parametrize("cfg", PRE)
def test_offsets_preshuffled_every_config(F, config_env, cfg):
    # pre-shuffled weights need N % 32 == 0 and K % 64 == 0
    offs = np.array([100, 100, 357, 500], np.int32)
    w = wl.make_stacked([520, 0, 0, 0], 512, 320, seed=530)
    config_env(cfg)
    print(f"case offsets pre cfg={cfg}", flush=True)
    ref = oracle.grouped_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, offs)
    P.assert_rows_match(run_offsets(F, w, offs, pre=True), ref, label=f"offsets pre cfg{cfg}")


def test_offsets_poisoned_unread_rows(F, config_env):
    """NaN codes and scales in rows past the last offset and in an empty group's
    weights: nothing may read them."""
    for cfg in PLAIN:
        config_env(cfg)
        w = wl.make_stacked([150, 0, 0], 136, 144, seed=540 + cfg)
        offs = np.array([40, 40, 117], np.int32)
        w.XQ[117:] = 0x7F
        w.x_scale[117:] = np.nan
        w.WQ[1] = 0xFF
        w.w_scale[1] = np.nan
        print(f"case offsets poison cfg={cfg}", flush=True)
        ref = oracle.grouped_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, offs)
        P.assert_rows_match(run_offsets(F, w, offs), ref, label=f"offsets poison cfg{cfg}")


@pytest.mark.parametrize("cfg,tail", [(16, None), (16, 2), (17, None), (26, None)])
def test_offsets_persistent_with_quarter_tail(F, config_env, cfg, tail):
    """A shape whose last round of 256x256 (or 128x256) tiles is partial."""
    sizes = [1000, 0, 733, 1300, 21]
    offs = np.cumsum(sizes).astype(np.int32)
    w = wl.make_stacked(sizes, 4096, 1024, seed=560 + cfg)
    config_env(cfg, tail)
    pre = cfg == 26
    print(f"case offsets persistent cfg={cfg} tail={tail}", flush=True)
    ref = oracle.grouped_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, offs)
    got = run_offsets(F, w, offs, pre=pre)
    P.assert_rows_match(got, ref, label=f"offsets persistent cfg{cfg}")
    assert np.array_equal(run_stacked(F, w, pre=pre), got)


# ---------------------------------------------------------------------------
# batched
# ---------------------------------------------------------------------------

BATCHED_EDGES = [
    # (G, M, N, K)
    (3, 1, 136, 16),
    (2, 63, 264, 112),
    (4, 129, 56, 144),
    (2, 300, 520, 1040),
    (1, 256, 1000, 320),
    (5, 33, 8, 208),
]


@pytest.mark.parametrize("cfg", PLAIN)
@pytest.mark.parametrize("case", range(len(BATCHED_EDGES)))
def test_batched_edges_every_config(F, config_env, cfg, case):
    G, M, N, K = BATCHED_EDGES[case]
    d = batched_case(G, M, N, K, 600 + case)
    config_env(cfg)
    print(f"case batched cfg={cfg} G={G} M={M} N={N} K={K}", flush=True)
    ref = oracle.grouped_batched(d.XQ, d.WQ, d.x_scale, d.w_scale)
    P.assert_rows_match(run_batched(F, d), ref, label=f"batched cfg{cfg}/case{case}")


@pytest.mark.parametrize("cfg", PRE)
def test_batched_preshuffled_every_config(F, config_env, cfg):
    d = batched_case(3, 129, 512, 256, 630)
    config_env(cfg)
    print(f"case batched pre cfg={cfg}", flush=True)
    ref = oracle.grouped_batched(d.XQ, d.WQ, d.x_scale, d.w_scale)
    P.assert_rows_match(run_batched(F, d, pre=True), ref, label=f"batched pre cfg{cfg}")


@pytest.mark.parametrize("cfg,tail", [(16, None), (16, 1), (17, 2), (26, None)])
def test_batched_persistent_equals_stacked(F, config_env, cfg, tail):
    """6 slabs of 768 rows: 288 tiles of 256x256, a partial last round.  Against the
    oracle, and bitwise against the stacked layout on the flattened slabs."""
    G, M, N, K = 6, 768, 4096, 1024
    d = batched_case(G, M, N, K, 640 + cfg)
    config_env(cfg, tail)
    pre = cfg == 26
    print(f"case batched persistent cfg={cfg} tail={tail}", flush=True)
    ref = oracle.grouped_batched(d.XQ, d.WQ, d.x_scale, d.w_scale)
    got = run_batched(F, d, pre=pre)
    P.assert_rows_match(got, ref, label=f"batched persistent cfg{cfg}")
    s = wl.Stacked(XQ=d.XQ.reshape(G * M, K), WQ=d.WQ, x_scale=d.x_scale.reshape(-1), w_scale=d.w_scale,
                   M_sizes=np.full(G, M, np.int64))
    assert np.array_equal(run_stacked(F, s, pre=pre), got.reshape(G * M, N))


def test_batched_default_plan_on_the_dense_expert_shape(F):
    p = F.plan(F.LAYOUT_BATCHED, False, 4, 512, 8192, 28672)
    assert p["persistent"] == 1 and p["m_tiles"] == 8
