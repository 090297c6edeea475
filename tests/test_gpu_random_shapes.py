"""GPU parity on seeded random shapes.

The edge-case lists elsewhere pick their shapes by hand; these cases draw them: a
layout (stacked, offsets, batched, padded with either zeroing flag, each with plain
or pre-shuffled W where the layout takes it, n_offsets, k_offsets, block-scaled
stacked; and, in a second set, block scales on the stacked, offsets, batched and
padded layouts with plain or pre-shuffled W), a group count, group sizes with empty
groups, N and K off every tile multiple (whole 128-wide blocks under block scales),
and either the default configuration or a forced one drawn from those the planner
accepts.  A third set draws larger shapes (up to 16 groups of up to 1500 rows, N and
K up to 2048) under the default selector, so that the persistent grid runs several
rounds with its quarter tiles and remainder modes.  Every case is compared with the oracle element by element, with
the sentinel and guard-band checks of the other parity tests.  The draws are fixed
by the case number, so a failure names a reproducible shape.
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

KINDS = ["stacked", "stacked_pre", "offsets", "offsets_pre", "batched", "padded", "padded_pre",
         "n_offsets", "k_offsets", "blockscale"]
N_CASES = 200


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp8_rowwise_scaled_amd as F
    F.load()
    return F


@contextmanager
def env(name, value):
    old = os.environ.get(name)
    if value is None:
        os.environ.pop(name, None)
    else:
        os.environ[name] = str(value)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop(name, None)
        else:
            os.environ[name] = old


def accepted_configs(F, layout, pre):
    """Configuration ids the planner accepts for a layout (as the other tests force them)."""
    from fp8_rowwise_scaled_amd import _lib
    ids = []
    for c in range(_lib.load().f8f8bf16_num_configs()):
        with env("FP8GG_CONFIG", c):
            try:
                F.plan(layout, pre, 2, 64, 64, 128)
                ids.append(c)
            except ValueError:
                pass
    return ids


def sizes_with_empties(rng, G, hi):
    s = rng.integers(0, hi + 1, G).astype(np.int64)
    s[rng.random(G) < 0.2] = 0
    return s


def run_packed(F, w, kind, offsets=None):
    whole, out = P.guarded_output((w.total_M, w.N))
    pre = kind.endswith("_pre")
    W = P.dev(w.WQ)
    if pre:
        W = F.f8f8bf16_shuffle_b(W)
    if kind.startswith("stacked"):
        fn = F.f8f8bf16_rowwise_grouped_stacked_preshuffle if pre else F.f8f8bf16_rowwise_grouped_stacked
        fn(P.dev(w.XQ), W, P.dev(w.x_scale), P.dev(w.w_scale), P.dev(w.M_sizes), out=out)
    else:
        fn = F.f8f8bf16_rowwise_grouped_offsets_preshuffle if pre else F.f8f8bf16_rowwise_grouped_offsets
        fn(P.dev(w.XQ), W, P.dev(w.x_scale), P.dev(w.w_scale), P.dev(np.asarray(offsets, np.int32)), out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(out)


def draw(case):
    """(kind, parameters) for one case, from the case number alone."""
    rng = np.random.default_rng(12000 + case)
    kind = KINDS[case % len(KINDS)]
    G = int(rng.integers(1, 9))
    pre = kind.endswith("_pre")
    if pre:
        N = 32 * int(rng.integers(1, 36))
        K = 64 * int(rng.integers(1, 18))
    elif kind == "blockscale":
        N = 128 * int(rng.integers(1, 6))
        K = 128 * int(rng.integers(1, 7))
    else:
        N = 8 * int(rng.integers(1, 140))
        K = 16 * int(rng.integers(1, 70))
    return rng, kind, G, N, K


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_shape_matches_oracle(F, case):
    rng, kind, G, N, K = draw(case)
    seed = 12500 + case
    use_default = rng.random() < 0.35
    if kind in ("stacked", "stacked_pre", "offsets", "offsets_pre"):
        layout = F.LAYOUT_STACKED if kind.startswith("stacked") else F.LAYOUT_OFFSETS
        sizes = sizes_with_empties(rng, G, 300)
        extra = int(rng.integers(0, 20)) if rng.random() < 0.3 else 0
        w = wl.make_stacked(sizes, N, K, seed=seed, total_M=int(sizes.sum()) + extra)
        cfgs = accepted_configs(F, layout, kind.endswith("_pre"))
        cfg = None if use_default else int(rng.choice(cfgs))
        print(f"case {case}: {kind} G={G} sizes={sizes.tolist()} extra={extra} N={N} K={K} cfg={cfg}", flush=True)
        offsets = np.cumsum(sizes).astype(np.int32)
        ref = (oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes) if kind.startswith("stacked")
               else oracle.grouped_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, offsets))
        with env("FP8GG_CONFIG", cfg):
            got = run_packed(F, w, kind, offsets)
        P.assert_rows_match(got, ref, label=f"case {case}")
    elif kind in ("padded", "padded_pre", "batched"):
        pre = kind == "padded_pre"
        em = int(rng.integers(1, 300))
        if kind == "batched":
            z = np.full(G, em, np.int64)
        else:
            z = rng.integers(0, em + 1, G).astype(np.int64)
            z[rng.random(G) < 0.2] = 0
        zeroing = bool(rng.random() < 0.5)
        d = wl.make_dynamic(z, em, N, K, seed=seed)
        layout = F.LAYOUT_BATCHED if kind == "batched" else F.LAYOUT_PADDED
        cfgs = accepted_configs(F, layout, pre)
        cfg = None if use_default else int(rng.choice(cfgs))
        print(f"case {case}: {kind} G={G} em={em} valid={z.tolist()} zeroing={zeroing} N={N} K={K} cfg={cfg}",
              flush=True)
        whole, out = P.guarded_output((G, em, N))
        W = F.f8f8bf16_shuffle_b(P.dev(d.WQ)) if pre else P.dev(d.WQ)
        with env("FP8GG_CONFIG", cfg):
            if kind == "batched":
                F.f8f8bf16_rowwise_grouped_batched(P.dev(d.XQ), W, P.dev(d.x_scale), P.dev(d.w_scale), out=out)
                ref = oracle.grouped_batched(d.XQ, d.WQ, d.x_scale, d.w_scale)
            else:
                fn = F.f8f8bf16_rowwise_grouped_dynamic_preshuffle if pre else F.f8f8bf16_rowwise_grouped_dynamic
                fn(P.dev(d.XQ), W, P.dev(d.x_scale), P.dev(d.w_scale), P.dev(d.zero_start_index_M),
                   zeroing_output_tensor=zeroing, out=out)
                ref = oracle.grouped_dynamic(d.XQ, d.WQ, d.x_scale, d.w_scale, d.zero_start_index_M, zeroing)
            torch.cuda.synchronize()
        P.check_guards(whole)
        P.assert_rows_match(P.bits_of(out).reshape(G * em, N), ref, label=f"case {case}")
    elif kind == "n_offsets":
        from tests.test_gpu_ragged import assert_cols_match
        M = int(rng.integers(1, 300))
        widths = 8 * rng.integers(0, 40, G)
        widths[rng.random(G) < 0.2] = 0
        trailing = 8 * int(rng.integers(0, 4))
        w = wl.make_n_offsets(widths, M, K, seed=seed, total_N=int(widths.sum()) + trailing + (8 if widths.sum() == 0 else 0))
        cfg = None if use_default else int(rng.choice([2, 7, 9, 18, 21, 28]))
        offs = np.cumsum(widths).astype(np.int32)
        print(f"case {case}: n_offsets G={G} M={M} widths={widths.tolist()} total_N={w.WQ.shape[0]} K={K} cfg={cfg}",
              flush=True)
        ref = oracle.grouped_n_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, offs)
        whole, y = P.guarded_output((M, w.WQ.shape[0]))
        with env("FP8GG_CONFIG", cfg):
            F.f8f8bf16_rowwise_grouped_n_offsets(P.dev(w.XQ), P.dev(w.WQ), P.dev(w.x_scale), P.dev(w.w_scale),
                                                 P.dev(offs), out=y)
            torch.cuda.synchronize()
        P.check_guards(whole)
        assert_cols_match(P.bits_of(y), ref, f"case {case}")
    elif kind == "k_offsets":
        M = int(rng.integers(1, 300))
        lengths = 16 * rng.integers(0, 40, G)
        lengths[rng.random(G) < 0.2] = 0
        total_K = int(lengths.sum()) + (16 if lengths.sum() == 0 else 0)
        w = wl.make_k_offsets(lengths, M, N, seed=seed, total_K=total_K)
        cfg = None if use_default else int(rng.choice([2, 7, 9, 18, 21, 28]))
        offs = np.cumsum(lengths).astype(np.int32)
        print(f"case {case}: k_offsets G={G} M={M} N={N} lengths={lengths.tolist()} cfg={cfg}", flush=True)
        ref = oracle.grouped_k_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, offs)
        whole, y = P.guarded_output((G, M, N))
        with env("FP8GG_CONFIG", cfg):
            F.f8f8bf16_rowwise_grouped_k_offsets(P.dev(w.XQ), P.dev(w.WQ), P.dev(w.x_scale), P.dev(w.w_scale),
                                                 P.dev(offs), out=y)
            torch.cuda.synchronize()
        P.check_guards(whole)
        P.assert_rows_match(P.bits_of(y).reshape(G * M, N), ref, label=f"case {case}")
    else:  # blockscale
        sizes = sizes_with_empties(rng, G, 300)
        w = wl.make_stacked_blockscale(sizes, N, K, seed=seed)
        cfg = None if use_default else int(rng.integers(0, 3))
        print(f"case {case}: blockscale G={G} sizes={sizes.tolist()} N={N} K={K} cfg={cfg}", flush=True)
        ref = oracle.grouped_stacked_blockscale(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
        total_M = int(sizes.sum())
        whole, y = P.guarded_output((total_M, N))
        with env("FP8GG_BS_CONFIG", cfg):
            F.f8f8bf16_groupwise_grouped_stacked(P.dev(w.XQ), P.dev(w.WQ), P.dev(w.x_scale), P.dev(w.w_scale),
                                                 P.dev(w.M_sizes), out=y)
            torch.cuda.synchronize()
        P.check_guards(whole)
        P.assert_rows_match(P.bits_of(y), ref, label=f"case {case}")


BS_KINDS = ["stacked", "stacked_pre", "offsets", "offsets_pre", "batched", "batched_pre", "padded", "padded_pre"]
N_BS_CASES = 64


def run_blockscale(F, kind, XQ, WQ, xs, ws, meta, out_shape, zeroing=True):
    """One block-scaled call on device copies; returns the output bits (guards checked)."""
    pre = kind.endswith("_pre")
    base = kind[:-4] if pre else kind
    whole, y = P.guarded_output(out_shape)
    W = F.f8f8bf16_shuffle_b(P.dev(WQ)) if pre else P.dev(WQ)
    fn = getattr(F, f"f8f8bf16_groupwise_grouped_{'dynamic' if base == 'padded' else base}"
                    + ("_preshuffle" if pre else ""))
    if base == "batched":
        fn(P.dev(XQ), W, P.dev(xs), P.dev(ws), out=y)
    elif base == "padded":
        fn(P.dev(XQ), W, P.dev(xs), P.dev(ws), P.dev(meta), zeroing_output_tensor=zeroing, out=y)
    else:
        fn(P.dev(XQ), W, P.dev(xs), P.dev(ws), P.dev(meta), out=y)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(y)


@pytest.mark.parametrize("case", range(N_BS_CASES))
def test_random_blockscale_matches_oracle(F, case):
    """Block scales on every layout, plain or pre-shuffled W: random group counts and
    sizes (empty groups included), N and K whole 128-wide blocks, the default or a
    forced tile configuration (the persistent one only where the layout takes it)."""
    rng = np.random.default_rng(13000 + case)
    kind = BS_KINDS[case % len(BS_KINDS)]
    base = kind[:-4] if kind.endswith("_pre") else kind
    G = int(rng.integers(1, 9))
    N = 128 * int(rng.integers(1, 6))
    K = 128 * int(rng.integers(1, 7))
    seed = 13500 + case
    cfg = None if rng.random() < 0.35 else int(rng.integers(0, 2 if base == "padded" else 3))
    if base in ("stacked", "offsets"):
        sizes = sizes_with_empties(rng, G, 300)
        w = wl.make_stacked_blockscale(sizes, N, K, seed=seed)
        offs = np.cumsum(sizes).astype(np.int32)
        print(f"case bs{case}: {kind} G={G} sizes={sizes.tolist()} N={N} K={K} cfg={cfg}", flush=True)
        if base == "stacked":
            ref = oracle.grouped_stacked_blockscale(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
            meta = w.M_sizes
        else:
            ref = oracle.grouped_offsets_blockscale(w.XQ, w.WQ, w.x_scale, w.w_scale, offs)
            meta = offs
        with env("FP8GG_BS_CONFIG", cfg):
            got = run_blockscale(F, kind, w.XQ, w.WQ, w.x_scale, w.w_scale, meta, (int(sizes.sum()), N))
        P.assert_rows_match(got, ref, label=f"case bs{case}")
    else:
        em = int(rng.integers(1, 300))
        if base == "batched":
            z = np.full(G, em, np.int64)
        else:
            z = rng.integers(0, em + 1, G).astype(np.int64)
            z[rng.random(G) < 0.2] = 0
        zeroing = bool(rng.random() < 0.5)
        d = wl.make_dynamic_blockscale(z, em, N, K, seed=seed)
        print(f"case bs{case}: {kind} G={G} em={em} valid={z.tolist()} zeroing={zeroing} N={N} K={K} cfg={cfg}",
              flush=True)
        if base == "batched":
            ref = oracle.grouped_batched_blockscale(d.XQ, d.WQ, d.x_scale, d.w_scale)
        else:
            ref = oracle.grouped_dynamic_blockscale(d.XQ, d.WQ, d.x_scale, d.w_scale, d.zero_start_index_M, zeroing)
        with env("FP8GG_BS_CONFIG", cfg):
            got = run_blockscale(F, kind, d.XQ, d.WQ, d.x_scale, d.w_scale, d.zero_start_index_M, (G, em, N),
                                 zeroing)
        P.assert_rows_match(got.reshape(G * em, N), ref, label=f"case bs{case}")


LARGE_KINDS = ["stacked", "stacked_pre", "offsets", "offsets_pre", "batched", "batched_pre", "padded", "padded_pre"]
N_LARGE_CASES = 24


@pytest.mark.parametrize("case", range(N_LARGE_CASES))
def test_random_large_shape_matches_oracle(F, case):
    """Larger shapes under the default selector: up to 16 groups of up to 1500 rows
    (slabs of up to 1200), N and K up to 2048, so the persistent grid runs several
    rounds and its quarter tiles (with the remainder mode sometimes forced)."""
    rng = np.random.default_rng(50000 + case)
    kind = LARGE_KINDS[case % len(LARGE_KINDS)]
    pre = kind.endswith("_pre")
    base = kind[:-4] if pre else kind
    G = int(rng.integers(1, 17))
    N = (32 if pre else 8) * int(rng.integers(1, (2048 // (32 if pre else 8)) + 1))
    K = (64 if pre else 16) * int(rng.integers(1, (2048 // (64 if pre else 16)) + 1))
    tail = None if rng.random() < 0.6 else int(rng.integers(0, 3))
    seed = 60000 + case
    with env("FP8GG_TAIL", tail):
        if base in ("stacked", "offsets"):
            sizes = rng.integers(0, 1500, G).astype(np.int64)
            sizes[rng.random(G) < 0.15] = 0
            w = wl.make_stacked(sizes, N, K, seed=seed)
            print(f"case large{case}: {kind} G={G} sizes={sizes.tolist()} N={N} K={K} tail={tail}", flush=True)
            offsets = np.cumsum(sizes).astype(np.int32)
            ref = (oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes) if base == "stacked"
                   else oracle.grouped_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, offsets))
            got = run_packed(F, w, kind, offsets)
            P.assert_rows_match(got, ref, label=f"large case {case}")
            return
        em = int(rng.integers(1, 1200))
        z = np.full(G, em, np.int64) if base == "batched" else rng.integers(0, em + 1, G).astype(np.int64)
        zeroing = bool(rng.random() < 0.5)
        d = wl.make_dynamic(z, em, N, K, seed=seed)
        print(f"case large{case}: {kind} G={G} em={em} valid={z.tolist()} zeroing={zeroing} N={N} K={K} "
              f"tail={tail}", flush=True)
        whole, out = P.guarded_output((G, em, N))
        W = F.f8f8bf16_shuffle_b(P.dev(d.WQ)) if pre else P.dev(d.WQ)
        if base == "batched":
            fn = F.f8f8bf16_rowwise_grouped_batched_preshuffle if pre else F.f8f8bf16_rowwise_grouped_batched
            fn(P.dev(d.XQ), W, P.dev(d.x_scale), P.dev(d.w_scale), out=out)
            ref = oracle.grouped_batched(d.XQ, d.WQ, d.x_scale, d.w_scale)
        else:
            fn = F.f8f8bf16_rowwise_grouped_dynamic_preshuffle if pre else F.f8f8bf16_rowwise_grouped_dynamic
            fn(P.dev(d.XQ), W, P.dev(d.x_scale), P.dev(d.w_scale), P.dev(d.zero_start_index_M),
               zeroing_output_tensor=zeroing, out=out)
            ref = oracle.grouped_dynamic(d.XQ, d.WQ, d.x_scale, d.w_scale, d.zero_start_index_M, zeroing)
        torch.cuda.synchronize()
        P.check_guards(whole)
        P.assert_rows_match(P.bits_of(out).reshape(G * em, N), ref, label=f"large case {case}")
