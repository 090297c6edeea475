"""GPU parity with many groups.

The device-side group lookup reads the per-group metadata eight groups at a time
and carries a running row prefix from one chunk to the next; the persistent grid
counts its tiles the same way.  These cases use 130 groups (17 chunks, the last
one partial), a tenth of them empty, on every layout that takes per-group
metadata, on the data-parallel, persistent, small-M and block-scaled kernels, and
calls whose tiles make more than one persistent round.  Each is compared with the
oracle element by element; offsets and stacked, and padded and stacked on the
compacted rows, are also compared bitwise.
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

G = 130


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp8_rowwise_scaled_amd as F
    F.load()
    return F


@contextmanager
def env(**values):
    saved = {k: os.environ.get(k) for k in values}
    try:
        for k, v in values.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = str(v)
        yield
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def sizes_with_empties(seed, hi):
    """G row counts in [1, hi], every tenth group (and group 0) empty."""
    s = np.random.default_rng(seed).integers(1, hi + 1, G).astype(np.int64)
    s[::10] = 0
    return s


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


def run_offsets(F, w, pre=False):
    whole, out = P.guarded_output((w.total_M, w.N))
    W = P.dev(w.WQ)
    fn = F.f8f8bf16_rowwise_grouped_offsets
    if pre:
        W = F.f8f8bf16_shuffle_b(W)
        fn = F.f8f8bf16_rowwise_grouped_offsets_preshuffle
    offs = torch.from_numpy(np.cumsum(w.M_sizes).astype(np.int32)).cuda()
    fn(P.dev(w.XQ), W, P.dev(w.x_scale), P.dev(w.w_scale), offs, out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(out)


def run_dynamic(F, d, zeroing=True):
    whole, out = P.guarded_output((d.G, d.expected_m, d.N))
    F.f8f8bf16_rowwise_grouped_dynamic(P.dev(d.XQ), P.dev(d.WQ), P.dev(d.x_scale), P.dev(d.w_scale),
                                       P.dev(d.zero_start_index_M), zeroing_output_tensor=zeroing, out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(out)


@pytest.fixture(scope="module")
def small_groups():
    """130 groups of 0..40 rows (2 477 rows); N = 264 and K = 272 leave an
    N tail on every tile width and a K tail on 128-byte stages."""
    return wl.make_stacked(sizes_with_empties(9100, 40), 264, 272, seed=9100)


# default selection, data-parallel 256x256 / 128x256 / 32x128 / 32x64, the
# persistent 256x256 and 128x256 grids, and the small-M register kernels
@pytest.mark.parametrize("cfg", [None, 0, 9, 20, 21, 16, 17, 15, 13])
def test_stacked_many_groups(F, small_groups, cfg):
    w = small_groups
    print(f"case many-groups stacked cfg={cfg}", flush=True)
    ref = oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
    with env(FP8GG_CONFIG=cfg):
        got = run_stacked(F, w)
    P.assert_rows_match(got, ref, label=f"stacked G={G} cfg={cfg}")


@pytest.mark.parametrize("cfg", [None, 16])
def test_offsets_many_groups_equal_stacked(F, small_groups, cfg):
    w = small_groups
    print(f"case many-groups offsets cfg={cfg}", flush=True)
    ref = oracle.grouped_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, np.cumsum(w.M_sizes).astype(np.int32))
    with env(FP8GG_CONFIG=cfg):
        got = run_offsets(F, w)
        stacked = run_stacked(F, w)
    P.assert_rows_match(got, ref, label=f"offsets G={G} cfg={cfg}")
    assert np.array_equal(got, stacked)


@pytest.mark.parametrize("cfg", [None, 26, 25, 4, 6, 27])
def test_stacked_preshuffled_many_groups(F, cfg):
    """Pre-shuffled W needs N % 32 == 0 and K % 64 == 0."""
    w = wl.make_stacked(sizes_with_empties(9200, 40), 256, 320, seed=9200)
    print(f"case many-groups stacked preshuffled cfg={cfg}", flush=True)
    ref = oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
    with env(FP8GG_CONFIG=cfg):
        got = run_stacked(F, w, pre=True)
    P.assert_rows_match(got, ref, label=f"stacked pre G={G} cfg={cfg}")


@pytest.mark.parametrize("cfg", [None, 9, 20])
@pytest.mark.parametrize("zeroing", [True, False])
def test_padded_many_slabs(F, cfg, zeroing):
    """130 slabs of 48 rows; the valid rows of each slab compared bitwise with the
    stacked entry point on the compacted rows."""
    z = np.random.default_rng(9300).integers(0, 49, G).astype(np.int64)
    z[::10] = 0
    z[1] = 48
    d = wl.make_dynamic(z, 48, 264, 272, seed=9300)
    print(f"case many-groups padded cfg={cfg} zeroing={zeroing}", flush=True)
    ref = oracle.grouped_dynamic(d.XQ, d.WQ, d.x_scale, d.w_scale, d.zero_start_index_M, zeroing)
    with env(FP8GG_CONFIG=cfg):
        got = run_dynamic(F, d, zeroing)
        got = got.reshape(G, 48, d.N)
        s = wl.Stacked(np.concatenate([d.XQ[g, :z[g]] for g in range(G)]), d.WQ,
                       np.concatenate([d.x_scale[g, :z[g]] for g in range(G)]), d.w_scale, z.copy())
        ys = run_stacked(F, s)
    P.assert_rows_match(got.reshape(-1, d.N), ref, label=f"padded G={G} cfg={cfg}")
    assert np.array_equal(np.concatenate([got[g, :z[g]] for g in range(G)]).reshape(ys.shape), ys)


@pytest.mark.parametrize("cfg,pre,tail", [(16, False, None), (16, False, 2), (26, True, None), (17, False, 2)])
def test_persistent_rounds_many_groups(F, cfg, pre, tail):
    """130 groups of up to 600 rows (34 784 rows) with N = 512: 400 tiles of 256x256
    (656 of 128x256), so the persistent grid walks a whole round and a partial
    second one, as whole tiles or (forced) as quarter tiles.  Against the oracle and
    bitwise against the data-parallel kernel with the same K order."""
    w = wl.make_stacked(sizes_with_empties(9400, 600), 512, 128, seed=9400)
    print(f"case many-groups persistent cfg={cfg} tail={tail} rows={int(w.M_sizes.sum())}", flush=True)
    ref = oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
    with env(FP8GG_CONFIG=cfg, FP8GG_TAIL=tail):
        got = run_stacked(F, w, pre=pre)
    P.assert_rows_match(got, ref, label=f"persistent G={G} cfg={cfg} tail={tail}")
    with env(FP8GG_CONFIG=4 if pre else 9):
        assert np.array_equal(run_stacked(F, w, pre=pre), got)


@pytest.mark.parametrize("cfg", [None, 0, 1, 2])
def test_blockscale_many_groups(F, cfg):
    w = wl.make_stacked_blockscale(sizes_with_empties(9500, 40), 256, 256, seed=9500)
    print(f"case many-groups blockscale cfg={cfg}", flush=True)
    ref = oracle.grouped_stacked_blockscale(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
    total_M = int(w.M_sizes.sum())
    whole, y = P.guarded_output((total_M, w.N))
    with env(FP8GG_BS_CONFIG=cfg):
        F.f8f8bf16_groupwise_grouped_stacked(P.dev(w.XQ), P.dev(w.WQ), P.dev(w.x_scale), P.dev(w.w_scale),
                                             P.dev(w.M_sizes), out=y)
        torch.cuda.synchronize()
    P.check_guards(whole)
    P.assert_rows_match(P.bits_of(y), ref, label=f"blockscale G={G} cfg={cfg}")
