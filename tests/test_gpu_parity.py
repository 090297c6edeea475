"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Small and edge-case shapes, compared element by element over the whole output.
Each call's output is prefilled with a sentinel and surrounded by guard bands.
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
    F.load()  # raises if libfp8gg.so is missing: there is no fallback
    return F


def _configs(preshuffled: bool):
    """Ids of the compiled kernel configurations of one kind (plain or pre-shuffled),
    found by asking the host planner which ones it accepts."""
    import fp8_rowwise_scaled_amd as F
    from fp8_rowwise_scaled_amd import _lib
    ids = []
    old = os.environ.get("FP8GG_CONFIG")
    try:
        for c in range(_lib.load().f8f8bf16_num_configs()):
            os.environ["FP8GG_CONFIG"] = str(c)
            try:
                F.plan(F.LAYOUT_STACKED, preshuffled, 2, 64, 64, 128)
                ids.append(c)
            except ValueError:
                pass
    finally:
        if old is None:
            os.environ.pop("FP8GG_CONFIG", None)
        else:
            os.environ["FP8GG_CONFIG"] = old
    return ids


PLAIN_CONFIGS = _configs(False)
PRE_CONFIGS = _configs(True)


@pytest.fixture
def config_env():
    """Forces a kernel configuration for the duration of a test."""
    old = os.environ.get("FP8GG_CONFIG")

    def set_cfg(c):
        if c is None:
            os.environ.pop("FP8GG_CONFIG", None)
        else:
            os.environ["FP8GG_CONFIG"] = str(c)
    yield set_cfg
    if old is None:
        os.environ.pop("FP8GG_CONFIG", None)
    else:
        os.environ["FP8GG_CONFIG"] = old


def run_stacked(F, w, pre=False):
    whole, out = P.guarded_output((w.total_M, w.N))
    W = P.dev(w.WQ)
    if pre:
        W = F.f8f8bf16_shuffle_b(W)
        fn = F.f8f8bf16_rowwise_grouped_stacked_preshuffle
    else:
        fn = F.f8f8bf16_rowwise_grouped_stacked
    fn(P.dev(w.XQ), W, P.dev(w.x_scale), P.dev(w.w_scale), P.dev(w.M_sizes), out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(out)


def run_dynamic(F, w, zeroing=True, pre=False):
    whole, out = P.guarded_output((w.G, w.expected_m, w.N))
    W = P.dev(w.WQ)
    if pre:
        W = F.f8f8bf16_shuffle_b(W)
        fn = F.f8f8bf16_rowwise_grouped_dynamic_preshuffle
    else:
        fn = F.f8f8bf16_rowwise_grouped_dynamic
    fn(P.dev(w.XQ), W, P.dev(w.x_scale), P.dev(w.w_scale), P.dev(w.zero_start_index_M),
       zeroing_output_tensor=zeroing, out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(out)


def oracle_stacked(w):
    return oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)


def oracle_dynamic(w, zeroing=True):
    return oracle.grouped_dynamic(w.XQ, w.WQ, w.x_scale, w.w_scale, w.zero_start_index_M, zeroing)


# ---------------------------------------------------------------------------

def test_tiny_stacked_workload(F):
    w = wl.tiny_stacked()
    print(f"case tiny_stacked {w.M_sizes.tolist()} N={w.N} K={w.K}", flush=True)
    P.assert_rows_match(run_stacked(F, w), oracle_stacked(w), label="tiny")


STACKED_EDGES = [
    # (M_sizes, N, K, total_M or None)
    ([0, 1, 31, 32, 33], 136, 16, None),
    ([63, 64, 65, 0], 264, 112, None),
    ([127, 128, 129], 56, 144, None),
    ([255, 0, 256, 257], 1000, 320, None),
    ([3, 0, 0, 5], 8, 208, 20),
    ([300], 520, 1040, None),
]


@pytest.mark.parametrize("cfg", PLAIN_CONFIGS)
@pytest.mark.parametrize("case", range(len(STACKED_EDGES)))
def test_stacked_edges_every_config(F, config_env, cfg, case):
    sizes, N, K, total_M = STACKED_EDGES[case]
    config_env(cfg)
    w = wl.make_stacked(sizes, N, K, seed=100 + case, total_M=total_M)
    print(f"case stacked cfg={cfg} sizes={sizes} N={N} K={K} total_M={w.total_M}", flush=True)
    P.assert_rows_match(run_stacked(F, w), oracle_stacked(w), label=f"cfg{cfg}/case{case}")


PADDED_EDGES = [
    # (zero_start_index_M, expected_m, N, K)
    ([0, 5, 64, 100], 100, 264, 144),
    ([300, 0, 299, 257], 300, 56, 208),
    ([-3, 40, 1000], 40, 1000, 64),      # clamped: negative -> 0, beyond -> expected_m
    ([512, 128, 1, 0], 512, 8, 16),
]


@pytest.mark.parametrize("cfg", PLAIN_CONFIGS)
@pytest.mark.parametrize("case", range(len(PADDED_EDGES)))
@pytest.mark.parametrize("zeroing", [True, False])
def test_padded_edges_every_config(F, config_env, cfg, case, zeroing):
    zsi, em, N, K = PADDED_EDGES[case]
    config_env(cfg)
    w = wl.make_dynamic(zsi, em, N, K, seed=200 + case)
    print(f"case padded cfg={cfg} zsi={zsi} em={em} N={N} K={K} zeroing={zeroing}", flush=True)
    P.assert_rows_match(run_dynamic(F, w, zeroing), oracle_dynamic(w, zeroing), label=f"cfg{cfg}/case{case}")


def test_overread_single_signed_neighbours(F, config_env):
    """Alternate groups get constant single-signed data, so any read past a group's
    rows, a row's K end or the N end accumulates coherently and shows."""
    for cfg in PLAIN_CONFIGS:
        config_env(cfg)
        sizes = [37, 70, 5, 129, 0, 64]
        N, K = 264, 208
        w = wl.make_stacked(sizes, N, K, seed=300 + cfg)
        start = 0
        for g, s in enumerate(sizes):
            if g % 2 == 1:
                w.XQ[start:start + s] = 0x38      # +1.0
                w.WQ[g] = 0x7E                    # +448
            start += s
        print(f"case single-signed cfg={cfg}", flush=True)
        P.assert_rows_match(run_stacked(F, w), oracle_stacked(w), label=f"single-signed cfg{cfg}")


def test_poisoned_unread_regions(F, config_env):
    """NaN codes and NaN scales where nothing may be read: rows past sum(M_sizes),
    empty groups' weights, padding rows and their x_scale."""
    for cfg in PLAIN_CONFIGS:
        config_env(cfg)
        sizes = [40, 0, 77]
        w = wl.make_stacked(sizes, 136, 144, seed=400 + cfg, total_M=150)
        w.XQ[117:] = 0x7F
        w.x_scale[117:] = np.nan
        w.WQ[1] = 0xFF
        w.w_scale[1] = np.nan
        print(f"case poison stacked cfg={cfg}", flush=True)
        got = run_stacked(F, w)
        P.assert_rows_match(got, oracle_stacked(w), label=f"poison stacked cfg{cfg}")
        d = wl.make_dynamic([3, 0, 70], 70, 136, 144, seed=410 + cfg)
        for g, z in enumerate(d.zero_start_index_M.tolist()):
            d.XQ[g, z:] = 0x7F
            d.x_scale[g, z:] = np.nan
        d.WQ[1] = 0x7F
        print(f"case poison padded cfg={cfg}", flush=True)
        for zeroing in (True, False):
            P.assert_rows_match(run_dynamic(F, d, zeroing), oracle_dynamic(d, zeroing),
                                label=f"poison padded cfg{cfg} zeroing={zeroing}")


def test_deterministic(F):
    w = wl.make_stacked([100, 300, 0, 212], 1000, 1040, seed=500)
    a = run_stacked(F, w)
    b = run_stacked(F, w)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("cfg", PLAIN_CONFIGS)
def test_dynamic_equals_stacked_on_compacted_rows_bitwise(F, config_env, cfg):
    """Same kernel configuration on both sides: the padded call's valid rows equal the
    stacked call on the compacted rows, bit for bit."""
    config_env(cfg)
    d = wl.make_dynamic([17, 0, 256, 100], 256, 264, 208, seed=600)
    yd = run_dynamic(F, d).reshape(d.G, d.expected_m, d.N)
    z = d.zero_start_index_M
    s = wl.Stacked(np.concatenate([d.XQ[g, :z[g]] for g in range(d.G)]), d.WQ,
                   np.concatenate([d.x_scale[g, :z[g]] for g in range(d.G)]), d.w_scale, z.copy())
    ys = run_stacked(F, s)
    assert np.array_equal(np.concatenate([yd[g, :z[g]] for g in range(d.G)]), ys)


@pytest.mark.parametrize("cfg", PLAIN_CONFIGS)
def test_k_tail_equals_zero_padded_k_bitwise(F, config_env, cfg):
    """Same configuration: a K that stops mid-tile equals the same data zero-padded to
    a whole number of tiles, bit for bit."""
    config_env(cfg)
    w = wl.make_stacked([50, 130], 264, 144, seed=700)
    a = run_stacked(F, w)
    pad = 256 - 144
    w2 = wl.Stacked(np.concatenate([w.XQ, np.zeros((w.total_M, pad), np.uint8)], 1),
                    np.concatenate([w.WQ, np.zeros((w.G, w.N, pad), np.uint8)], 2),
                    w.x_scale, w.w_scale, w.M_sizes)
    b = run_stacked(F, w2)
    assert np.array_equal(a, b)


def test_identity_weights_reproduce_a(F):
    """B = I: with 1.0 on W's diagonal, w_scale = 1 and power-of-two x_scale the
    output is exactly dec(XQ) * x_scale (a lost accumulator slot would zero rows)."""
    K = 256
    rng = np.random.default_rng(800)
    XQ = rng.integers(0, 256, (96, K)).astype(np.uint8)
    XQ[(XQ & 0x7F) == 0x7F] = 0x38
    WQ = np.zeros((1, K, K), np.uint8)
    WQ[0, np.arange(K), np.arange(K)] = 0x38
    xs = (2.0 ** rng.integers(-3, 3, 96)).astype(np.float32)
    w = wl.Stacked(XQ, WQ, xs, np.ones((1, K), np.float32), np.array([96]))
    got = run_stacked(F, w)
    want = (torch.from_numpy(XQ).view(torch.float8_e4m3fn).float() * torch.from_numpy(xs)[:, None])
    want = want.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nz = (want & 0x7FFF) != 0
    assert np.array_equal(got[nz], want[nz])
    assert np.all((got[~nz] & 0x7FFF) == 0)


def test_k_zero_zero_fills_everything(F):
    w = wl.make_stacked([3, 4], 24, 0, seed=900, total_M=9)
    got = run_stacked(F, w)
    assert np.all(got == 0)
    d = wl.make_dynamic([1, 2], 3, 24, 0, seed=901)
    got = run_dynamic(F, d, zeroing=False)
    assert np.all(got == 0)


def test_metadata_clamping(F):
    w = wl.make_stacked([-5, 3, 1_000_000], 136, 144, seed=950, total_M=40)
    P.assert_rows_match(run_stacked(F, w), oracle_stacked(w), label="clamp stacked")


def test_refusals_raise(F):
    w = wl.make_stacked([3], 24, 32, seed=960)
    with pytest.raises(ValueError):   # K not a multiple of 16
        F.f8f8bf16_rowwise_grouped_stacked(P.dev(w.XQ[:, :24].copy()), P.dev(w.WQ[:, :, :24].copy()),
                                           P.dev(w.x_scale), P.dev(w.w_scale), P.dev(w.M_sizes))
    with pytest.raises(ValueError):   # strided output
        out = torch.empty((3, 48), dtype=torch.bfloat16, device="cuda")[:, :24]
        F.f8f8bf16_rowwise_grouped_stacked(P.dev(w.XQ), P.dev(w.WQ), P.dev(w.x_scale), P.dev(w.w_scale),
                                           P.dev(w.M_sizes), out=out)


# ---------------------------------------------------------------------------
# pre-shuffled weights
# ---------------------------------------------------------------------------

def shuffle_reference(WQ: np.ndarray) -> np.ndarray:
    """The pre-shuffled byte order stated in include/fp8gg.h, written with numpy:
    block (g, nb, kb) of 2048 bytes holds, at h*1024 + 16*l, the 16 bytes
    W[g, 32nb + perm32(l%32), 64kb + 32(l/32) + 16h .. +16)."""
    G, N, K = WQ.shape
    perm = np.array([16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3) for r in range(32)])
    assert sorted(perm) == list(range(32))
    v = WQ.reshape(G, N // 32, 32, K // 64, 2, 2, 16)      # g, nb, row, kb, l/32, h, byte
    v = v[:, :, perm]                                       # row slot r' holds row perm32(r')
    v = v.transpose(0, 1, 3, 5, 4, 2, 6)                    # g, nb, kb, h, l/32, r', byte
    return np.ascontiguousarray(v).reshape(G, N, K)


def test_shuffle_layout(F):
    rng = np.random.default_rng(1000)
    W = rng.integers(0, 256, (3, 96, 192)).astype(np.uint8)
    got = F.f8f8bf16_shuffle_b(P.dev(W)).cpu().numpy()
    assert np.array_equal(got, shuffle_reference(W))


PRE_CASES = [
    # (layout, sizes or zsi, expected_m, N, K)
    ("stacked", [0, 1, 31, 32, 33], None, 128, 64),
    ("stacked", [63, 64, 65, 0, 129], None, 288, 192),
    ("stacked", [300, 0, 77], None, 544, 1024),
    ("padded", [0, 5, 64, 100], 100, 256, 128),
    ("padded", [300, 0, 299, 257], 300, 96, 320),
]


@pytest.mark.parametrize("cfg", [None] + PRE_CONFIGS)
@pytest.mark.parametrize("case", range(len(PRE_CASES)))
def test_preshuffled_matches_oracle_and_plain(F, config_env, cfg, case):
    """Pre-shuffled vs oracle, and bitwise vs the plain LDS kernel of the same K order
    (configuration 0 accumulates the K steps in the same sequence)."""
    layout, meta, em, N, K = PRE_CASES[case]
    print(f"case preshuffle cfg={cfg} {layout} {meta} em={em} N={N} K={K}", flush=True)
    if layout == "stacked":
        w = wl.make_stacked(meta, N, K, seed=1100 + case)
        config_env(0)
        plain = run_stacked(F, w)
        config_env(cfg)
        got = run_stacked(F, w, pre=True)
        P.assert_rows_match(got, oracle_stacked(w), label=f"pre cfg{cfg} case{case}")
    else:
        w = wl.make_dynamic(meta, em, N, K, seed=1100 + case)
        config_env(0)
        plain = run_dynamic(F, w)
        config_env(cfg)
        got = run_dynamic(F, w, pre=True)
        P.assert_rows_match(got, oracle_dynamic(w), label=f"pre cfg{cfg} case{case}")
    assert np.array_equal(got, plain), "pre-shuffled and plain paths differ bitwise"


def test_preshuffled_refuses_partial_blocks(F):
    w = wl.make_stacked([4], 40, 64, seed=1200)
    with pytest.raises(ValueError):
        F.f8f8bf16_shuffle_b(P.dev(w.WQ))
    with pytest.raises(ValueError):
        F.f8f8bf16_rowwise_grouped_stacked_preshuffle(P.dev(w.XQ), P.dev(w.WQ), P.dev(w.x_scale),
                                                      P.dev(w.w_scale), P.dev(w.M_sizes))


def test_graph_replay_matches_eager(F):
    """Calls captured into a HIP graph and replayed several times, with eager work and
    synchronisation between replays, give the eager result every time."""
    ws = [wl.make_stacked([3, 0, 40, 1], 264, 208, seed=1300), wl.make_stacked([1, 0, 0, 0], 7168 // 4, 512,
                                                                                 seed=1301)]
    eager, graphs = [], []
    for w in ws:
        args = [P.dev(a) for a in (w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)]
        out = torch.empty((w.total_M, w.N), dtype=torch.bfloat16, device="cuda")
        F.f8f8bf16_rowwise_grouped_stacked(*args, out=out)
        torch.cuda.synchronize()
        eager.append(P.bits_of(out).copy())
        g = torch.cuda.CUDAGraph()
        gout = torch.empty_like(out)
        with torch.cuda.graph(g):
            F.f8f8bf16_rowwise_grouped_stacked(*args, out=gout)
        graphs.append((g, gout, args))
    for rep in range(4):
        for (g, gout, args), want in zip(graphs, eager):
            gout.view(torch.int16).fill_(P.SENTINEL)     # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(P.bits_of(gout), want), f"replay {rep} differs from eager"
