"""GPU closed forms: results the arithmetic fixes exactly, compared bit for bit.

One-hot rows.  A row of X whose only nonzero code is a at column k gives
Y[r, n] = dec(a) * dec(W[g, n, k]) * x_scale[r] * w_scale[g, n].  Two e4m3 values
have at most four significant bits each, so their product has at most eight and
is a bf16 value; with power-of-two scales every step is exact in fp32 and no
rounding happens anywhere.  Every configuration must return exactly that value
(a zero result with either sign).  A wrong K, row, column or group index in any
kernel changes the value picked, not just its last bits.  The expected values
decode the codes through torch's float8_e4m3fn type, not through the oracle.

Power-of-two scale changes.  Multiplying by two commutes with fp32 and bf16
rounding away from overflow and underflow, so doubling x_scale of some rows must
double exactly those output rows and leave every other bit unchanged, and halving
some of one group's w_scale entries must halve exactly those columns of that
group's rows.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from tests import parity as P
from tests.test_gpu_blockscale import forced as forced_bs
from tests.test_gpu_parity import PLAIN_CONFIGS, PRE_CONFIGS, config_env  # noqa: F401 (fixture)
from tests.test_gpu_ragged import RAGGED_CONFIGS, run_k, run_n
from tests.test_gpu_ragged import forced as forced_cfg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp8_rowwise_scaled_amd as F
    F.load()
    return F


def decode(codes: np.ndarray) -> np.ndarray:
    """e4m3fn codes -> float64 through torch's own float8 type."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.float().double().numpy()


def bf16_bits_exact(v: np.ndarray) -> np.ndarray:
    """Bits of float64 values that are bf16 values already (asserted), -0 as +0."""
    v = np.where(v == 0, 0.0, v)
    f = v.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32).astype(np.float64), v), "not a bf16 value"
    return b


def unsigned_zero(bits: np.ndarray) -> np.ndarray:
    return np.where(bits == 0x8000, np.uint16(0), bits)


FINITE_NONZERO = np.array([c for c in range(256) if c not in (0x00, 0x80, 0x7F, 0xFF)], np.uint8)


def one_hot(rng, rows, K):
    """X rows with one nonzero finite code each, at a random column (tail included)."""
    X = np.zeros((rows, K), np.uint8)
    ks = rng.integers(0, K, rows)
    codes = rng.choice(FINITE_NONZERO, rows)
    X[np.arange(rows), ks] = codes
    return X, ks, codes


def pow2(rng, shape, lo=-3, hi=3):
    return np.ldexp(1.0, rng.integers(lo, hi + 1, shape)).astype(np.float32)


def run_stacked(F, XQ, WQ, xs, ws, M_sizes, pre):
    whole, out = P.guarded_output((XQ.shape[0], WQ.shape[1]))
    W = P.dev(WQ)
    fn = F.f8f8bf16_rowwise_grouped_stacked
    if pre:
        W = F.f8f8bf16_shuffle_b(W)
        fn = F.f8f8bf16_rowwise_grouped_stacked_preshuffle
    fn(P.dev(XQ), W, P.dev(xs), P.dev(ws), P.dev(M_sizes), out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return P.bits_of(out)


def one_hot_stacked_case(rng, sizes, N, K):
    G, M = len(sizes), int(sum(sizes))
    XQ, ks, codes = one_hot(rng, M, K)
    WQ = rng.choice(np.arange(256, dtype=np.uint8)[[c not in (0x7F, 0xFF) for c in range(256)]], (G, N, K))
    xs, ws = pow2(rng, M), pow2(rng, (G, N))
    owner = np.repeat(np.arange(G), sizes)
    y = (decode(codes)[:, None] * decode(WQ[owner, :, ks]) * xs[:, None].astype(np.float64)
         * ws[owner].astype(np.float64))
    return XQ, WQ, xs, ws, np.array(sizes, np.int64), bf16_bits_exact(y)


@pytest.mark.parametrize("cfg", PLAIN_CONFIGS)
def test_one_hot_rows_exact_stacked(F, config_env, cfg):
    config_env(cfg)
    rng = np.random.default_rng(7000 + cfg)
    for sizes, N, K in (([37, 0, 90, 1], 200, 336), ([2, 1], 64, 1040)):
        print(f"case one-hot stacked cfg={cfg} sizes={sizes} N={N} K={K}", flush=True)
        XQ, WQ, xs, ws, Ms, want = one_hot_stacked_case(rng, sizes, N, K)
        got = unsigned_zero(run_stacked(F, XQ, WQ, xs, ws, Ms, pre=False))
        assert np.array_equal(got, want), f"cfg {cfg}: {int((got != want).sum())} elements differ"


@pytest.mark.parametrize("cfg", PRE_CONFIGS)
def test_one_hot_rows_exact_stacked_preshuffled(F, config_env, cfg):
    config_env(cfg)
    rng = np.random.default_rng(7100 + cfg)
    for sizes, N, K in (([37, 0, 90, 1], 192, 320), ([300, 5], 96, 1024)):
        print(f"case one-hot stacked pre cfg={cfg} sizes={sizes} N={N} K={K}", flush=True)
        XQ, WQ, xs, ws, Ms, want = one_hot_stacked_case(rng, sizes, N, K)
        got = unsigned_zero(run_stacked(F, XQ, WQ, xs, ws, Ms, pre=True))
        assert np.array_equal(got, want), f"cfg {cfg}: {int((got != want).sum())} elements differ"


@pytest.mark.parametrize("zeroing", [True, False])
def test_one_hot_rows_exact_padded(F, zeroing):
    """Default selector on the padded layout (whole slabs, empty and partial groups,
    N and K off the tile multiples): valid rows exact, padding rows zero or untouched."""
    rng = np.random.default_rng(7200 + zeroing)
    G, em, N, K = 5, 150, 264, 592
    z = np.array([150, 0, 37, 149, 1], np.int64)
    XQ = rng.integers(0, 256, (G, em, K), dtype=np.uint8)
    XQ[XQ == 0x7F] = 0x7E
    XQ[XQ == 0xFF] = 0xFE
    WQ = rng.integers(0, 256, (G, N, K), dtype=np.uint8)
    WQ[WQ == 0x7F] = 0x7E
    WQ[WQ == 0xFF] = 0xFE
    xs, ws = pow2(rng, (G, em)), pow2(rng, (G, N))
    want = np.zeros((G, em, N), np.uint16)
    for g in range(G):
        X1, ks, codes = one_hot(rng, int(z[g]), K)
        XQ[g, :z[g]] = X1
        y = decode(codes)[:, None] * decode(WQ[g][:, ks].T) * xs[g, :z[g], None].astype(np.float64) \
            * ws[g][None, :].astype(np.float64)
        want[g, :z[g]] = bf16_bits_exact(y)
    print(f"case one-hot padded zeroing={zeroing}", flush=True)
    whole, out = P.guarded_output((G, em, N))
    F.f8f8bf16_rowwise_grouped_dynamic(P.dev(XQ), P.dev(WQ), P.dev(xs), P.dev(ws), P.dev(z),
                                       zeroing_output_tensor=zeroing, out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    got = P.bits_of(out)
    for g in range(G):
        assert np.array_equal(unsigned_zero(got[g, :z[g]]), want[g, :z[g]]), f"group {g}: valid rows differ"
        pad = got[g, z[g]:]
        assert np.all(pad == 0) if zeroing else np.all(pad == np.uint16(P.SENTINEL)), f"group {g}: padding rows"


def as_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("cfg", PLAIN_CONFIGS)
def test_power_of_two_scale_changes_are_exact(F, config_env, cfg):
    config_env(cfg)
    w = wl.make_stacked([70, 0, 133, 3], 136, 272, seed=7300 + cfg)
    rng = np.random.default_rng(7300 + cfg)
    print(f"case scale doubling cfg={cfg}", flush=True)
    base = run_stacked(F, w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes, pre=False)

    rows = np.sort(rng.choice(w.total_M, 25, replace=False))
    xs2 = w.x_scale.copy()
    xs2[rows] *= 2
    got = run_stacked(F, w.XQ, w.WQ, xs2, w.w_scale, w.M_sizes, pre=False)
    other = np.setdiff1d(np.arange(w.total_M), rows)
    assert np.array_equal(got[other], base[other]), "rows whose scale did not change moved"
    assert np.array_equal(as_f32(got[rows]), 2 * as_f32(base[rows])), "doubled rows are not exactly doubled"

    g, cols = 2, np.sort(rng.choice(w.N, 40, replace=False))
    ws2 = w.w_scale.copy()
    ws2[g, cols] *= 0.5
    got = run_stacked(F, w.XQ, w.WQ, w.x_scale, ws2, w.M_sizes, pre=False)
    start = int(w.M_sizes[:g].sum())
    grows = np.arange(start, start + int(w.M_sizes[g]))
    mask = np.zeros(got.shape, bool)
    mask[np.ix_(grows, cols)] = True
    assert np.array_equal(got[~mask], base[~mask]), "entries whose scale did not change moved"
    assert np.array_equal(as_f32(got[mask]), 0.5 * as_f32(base[mask])), "halved entries are not exactly halved"


FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


@pytest.mark.parametrize("cfg", [None] + RAGGED_CONFIGS)
def test_one_hot_rows_exact_n_offsets(F, cfg):
    """n_offsets: column n of group g takes slab g of X, so Y[m, n] is the single
    product at slab g's one-hot column; columns of no group keep the sentinel."""
    rng = np.random.default_rng(7400 + (cfg or 0))
    G, M, K = 4, 70, 208
    widths = [0, 37, 200, 64]
    total_N = 304                                   # three trailing columns of no group
    offs = np.cumsum(widths).astype(np.int32)
    owner = np.full(total_N, -1)
    start = 0
    for g, wd in enumerate(widths):
        owner[start:start + wd] = g
        start += wd
    XQ = np.zeros((G, M, K), np.uint8)
    ks = rng.integers(0, K, (G, M))
    codes = rng.choice(FINITE_NONZERO, (G, M))
    gi, mi = np.meshgrid(np.arange(G), np.arange(M), indexing="ij")
    XQ[gi, mi, ks] = codes
    WQ = rng.choice(FINITE, (total_N, K))
    xs, ws = pow2(rng, (G, M)), pow2(rng, total_N)
    cols = np.nonzero(owner >= 0)[0]
    gc = owner[cols]
    y = (decode(codes[gc].T) * decode(WQ[cols[None, :], ks[gc].T]) * xs[gc].T.astype(np.float64)
         * ws[cols][None, :].astype(np.float64))
    want = bf16_bits_exact(y)
    print(f"case one-hot n_offsets cfg={cfg}", flush=True)
    with forced_cfg(cfg):
        got = run_n(F, XQ, WQ, xs, ws, offs)
    assert np.array_equal(unsigned_zero(got[:, cols]), want), "written columns differ"
    assert np.all(got[:, owner < 0] == np.uint16(P.SENTINEL)), "columns of no group were written"


@pytest.mark.parametrize("cfg", [None] + RAGGED_CONFIGS)
def test_one_hot_rows_exact_k_offsets(F, cfg):
    """k_offsets: the one-hot column of row m lies in exactly one group's K slice;
    that group's Y[g, m, :] is the single product, every other group's row is zero
    (an empty slice included)."""
    rng = np.random.default_rng(7500 + (cfg or 0))
    M, N = 70, 136
    widths = [0, 48, 400, 160]
    G, total_K = len(widths), sum(widths)
    offs = np.cumsum(widths).astype(np.int32)
    kowner = np.repeat(np.arange(G), widths)
    XQ, ks, codes = one_hot(rng, M, total_K)
    WQ = rng.choice(FINITE, (N, total_K))
    xs, ws = pow2(rng, (G, M)), pow2(rng, (G, N))
    y = np.zeros((G, M, N))
    gm = kowner[ks]
    y[gm, np.arange(M)] = (decode(codes)[:, None] * decode(WQ[:, ks].T) * xs[gm, np.arange(M)][:, None].astype(np.float64)
                           * ws[gm].astype(np.float64))
    want = bf16_bits_exact(y)
    print(f"case one-hot k_offsets cfg={cfg}", flush=True)
    with forced_cfg(cfg):
        got = run_k(F, XQ, WQ, xs, ws, offs)
    assert np.array_equal(unsigned_zero(got), want)


@pytest.mark.parametrize("cfg", [None, 0, 1, 2])
def test_one_hot_rows_exact_blockscale(F, cfg):
    """Block scales: the single product of row m lies in K block k_m // 128, so only
    x_scale[m, kb] and w_scale[g, n // 128, kb] of that block may reach Y[m, n]; with
    power-of-two block scales the result is exact."""
    rng = np.random.default_rng(7600 + (cfg or 0))
    sizes, N, K = [37, 0, 130, 3], 384, 640
    G, M = len(sizes), sum(sizes)
    XQ, ks, codes = one_hot(rng, M, K)
    WQ = rng.choice(FINITE, (G, N, K))
    xs, ws = pow2(rng, (M, K // 128)), pow2(rng, (G, N // 128, K // 128))
    owner = np.repeat(np.arange(G), sizes)
    kb = ks // 128
    y = (decode(codes)[:, None] * decode(WQ[owner, :, ks]) * xs[np.arange(M), kb][:, None].astype(np.float64)
         * ws[owner[:, None], (np.arange(N) // 128)[None, :], kb[:, None]].astype(np.float64))
    want = bf16_bits_exact(y)
    print(f"case one-hot block-scaled cfg={cfg}", flush=True)
    with forced_bs(cfg):
        whole, out = P.guarded_output((M, N))
        F.f8f8bf16_groupwise_grouped_stacked(P.dev(XQ), P.dev(WQ), P.dev(xs), P.dev(ws),
                                             P.dev(np.array(sizes, np.int64)), out=out)
        torch.cuda.synchronize()
    P.check_guards(whole)
    assert np.array_equal(unsigned_zero(P.bits_of(out)), want)
