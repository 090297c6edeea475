"""Pins for the CPU oracle: it is checked against things other than itself.

* the e4m3fn decode against torch's float8 type and the format definition;
* the fp64 -> bf16 rounding against torch's fp32 -> bf16 and hand-derived ties;
* the whole grouped GEMM against an exact rational brute force on tiny shapes and
  against a hand-derived worked example;
* invariants: summation-order independence, zero-padded K, the rowwise-scale
  factorisation, dynamic == stacked on the compacted rows, closed forms (B = I,
  one-hot rows, power-of-two scales), row classification;
* planted mistakes: each one is injected into the oracle and must trip a pin.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import grouped_gemm as og
from tests import exact_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FINITE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _rand_problem(seed, sizes, N, K, total_M=None, finite=True):
    rng = np.random.default_rng(seed)
    sizes = np.asarray(sizes, np.int64)
    if total_M is None:
        total_M = int(np.clip(sizes, 0, None).sum())
    G = sizes.size
    XQ = rng.choice(FINITE_CODES, size=(total_M, K)).astype(np.uint8)
    WQ = rng.choice(FINITE_CODES, size=(G, N, K)).astype(np.uint8)
    xs = (2.0 ** rng.uniform(-12, 4, total_M)).astype(np.float32)
    ws = (2.0 ** rng.uniform(-12, 4, (G, N))).astype(np.float32)
    return XQ, WQ, xs, ws, sizes


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def test_decode_matches_torch_all_codes():
    t = oracle.e4m3fn_table()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(t), nan)
    assert np.array_equal(t[~nan], ref[~nan])
    assert np.array_equal(np.signbit(t[~nan]), np.signbit(ref[~nan]))


def test_decode_golden_codes():
    n = 0
    for line in open(os.path.join(GOLDEN, "e4m3fn_codes.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code_s, val_s = line.split()[:2]
        code = int(code_s, 16)
        got = oracle.decode_e4m3fn(np.array([code], np.uint8))[0]
        if val_s == "nan":
            assert np.isnan(got), hex(code)
        else:
            want = float.fromhex(val_s) if "0x" in val_s else float(val_s)
            assert got == want and np.signbit(got) == np.signbit(want), (hex(code), got, want)
        n += 1
    assert n >= 15


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def test_bf16_golden_cases():
    n = 0
    for line in open(os.path.join(GOLDEN, "bf16_rne_cases.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        x_s, bits_s = line.split()[:2]
        x = float.fromhex(x_s)
        got = int(oracle.bf16_rne_from_f64(np.array([x]))[0])
        assert got == int(bits_s, 16), (x_s, hex(got), bits_s)
        n += 1
    assert n >= 15


def test_bf16_ulp_golden_cases():
    n = 0
    for line in open(os.path.join(GOLDEN, "bf16_ulp_cases.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        x_s, u_s = line.split()[:2]
        got = float(oracle.bf16_ulp(np.array([float.fromhex(x_s)]))[0])
        assert got == float.fromhex(u_s), (x_s, got.hex(), u_s)
        n += 1
    assert n >= 10


def _bf16_values_torch(bits):
    """bf16 bit patterns -> fp64 through torch's own bfloat16 type (not the oracle's
    bit shift)."""
    b = torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16).copy())
    return b.view(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_ulp_equals_successor_spacing():
    """bf16_ulp(|x|) is the distance between consecutive bf16 numbers around |x|:
    for every positive finite pattern b, the gap v(b + 1) - v(b) (values decoded by
    torch) must equal bf16_ulp at v(b), at random points strictly inside [v(b),
    v(b + 1)) and at -v(b); and above 2^-126 it must equal 2^16 times numpy's fp32
    spacing (fp32 has 16 more fraction bits)."""
    b = np.arange(0x0000, 0x7F7F, dtype=np.uint16)           # 0 .. the largest finite - 1
    v = _bf16_values_torch(b)
    gap = _bf16_values_torch(b + 1) - v
    assert np.array_equal(oracle.bf16_ulp(v), gap)
    assert np.array_equal(oracle.bf16_ulp(-v), gap)
    rng = np.random.default_rng(60)
    inside = v + gap * rng.uniform(0.0, 1.0, v.size)
    inside = np.where(inside < v + gap, inside, v)            # stay inside the half-open gap
    assert np.array_equal(oracle.bf16_ulp(inside), gap)
    normal = v >= 2.0 ** -126
    f32_step = np.spacing(v[normal].astype(np.float32)).astype(np.float64) * 2.0 ** 16
    assert np.array_equal(oracle.bf16_ulp(v[normal]), f32_step)


def test_planted_ulp_mistake_is_caught(monkeypatch):
    """A doubled ulp (it would silently widen every GPU tolerance) trips the pins."""
    orig = og.bf16_ulp
    for wrong in (lambda x: 2.0 * orig(x), lambda x: 0.5 * orig(x)):
        monkeypatch.setattr(og, "bf16_ulp", wrong)
        monkeypatch.setattr(oracle, "bf16_ulp", wrong)
        with pytest.raises(AssertionError):
            test_bf16_ulp_equals_successor_spacing()
        with pytest.raises(AssertionError):
            test_bf16_ulp_golden_cases()


def test_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[~np.isnan(x)]
    # plus values near bf16 rounding boundaries and in the subnormal range
    base = rng.standard_normal(50_000).astype(np.float32)
    b16 = torch.from_numpy(base).to(torch.bfloat16).float().numpy()
    ties = (b16.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    sub = (rng.standard_normal(20_000) * 2.0 ** -130).astype(np.float32)
    x = np.concatenate([x, ties, sub, np.float32([0.0, -0.0, np.inf, -np.inf])])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_rne_from_f64(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_exact_rational_agrees_on_random_fp64():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(3000) * 2.0 ** rng.integers(-140, 130, 3000)
    got = oracle.bf16_rne_from_f64(x)
    from fractions import Fraction
    want = np.array([exact_ref.bf16_bits_exact(Fraction(float(v))) for v in x], np.uint16)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# the grouped GEMM, end to end
# ---------------------------------------------------------------------------

def _check_bruteforce(seed, sizes, N, K, total_M=None):
    XQ, WQ, xs, ws, sizes = _rand_problem(seed, sizes, N, K, total_M)
    res = oracle.grouped_stacked(XQ, WQ, xs, ws, sizes)
    exact = exact_ref.stacked_exact(XQ, WQ, xs, ws, sizes)
    for r, row in enumerate(exact):
        if row is None:
            if res.row_class[r] != oracle.ROW_UNTOUCHED:
                return False
            continue
        if res.row_class[r] != oracle.ROW_WRITTEN:
            return False
        got = res.bits[r].astype(np.int64)
        want = np.array(row, np.int64)
        zero = (want & 0x7FFF) == 0
        if not np.array_equal(got[~zero], want[~zero]):
            return False
        if not np.all((got[zero] & 0x7FFF) == 0):
            return False
    return True


BRUTE_CASES = [
    (11, [2, 0, 3], 5, 48, None),
    (12, [1, 4], 3, 32, 7),
    (13, [0, 0, 2, 1], 6, 16, None),
    (14, [3], 4, 80, None),
]


@pytest.mark.parametrize("seed,sizes,N,K,total_M", BRUTE_CASES)
def test_stacked_equals_exact_bruteforce(seed, sizes, N, K, total_M):
    assert _check_bruteforce(seed, sizes, N, K, total_M)


def _rows_match_exact(res, exact):
    """res (an OracleResult over rows) against exact rows (None: no group)."""
    for r, row in enumerate(exact):
        if row is None:
            if res.row_class[r] != oracle.ROW_UNTOUCHED:
                return False
            continue
        if res.row_class[r] != oracle.ROW_WRITTEN:
            return False
        got = res.bits.reshape(len(exact), -1)[r].astype(np.int64)
        want = np.array(row, np.int64)
        zero = (want & 0x7FFF) == 0
        if not np.array_equal(got[~zero], want[~zero]):
            return False
        if not np.all((got[zero] & 0x7FFF) == 0):
            return False
    return True


# (seed, offsets, N, K, total_M): offsets are int32 inclusive prefix sums
OFFSETS_CASES = [
    (31, [2, 2, 5], 4, 48, None),      # an empty middle group
    (32, [0, 3, 3, 7], 3, 32, 9),      # rows 7 and 8 belong to no group
    (33, [4], 5, 16, None),
]


def _check_offsets(seed, offsets, N, K, total_M):
    sizes = np.diff([0] + offsets)
    XQ, WQ, xs, ws, _ = _rand_problem(seed, sizes, N, K, total_M)
    res = oracle.grouped_offsets(XQ, WQ, xs, ws, np.array(offsets, np.int32))
    return _rows_match_exact(res, exact_ref.offsets_exact(XQ, WQ, xs, ws, offsets))


@pytest.mark.parametrize("seed,offsets,N,K,total_M", OFFSETS_CASES)
def test_offsets_equals_exact_bruteforce(seed, offsets, N, K, total_M):
    assert _check_offsets(seed, offsets, N, K, total_M)


def test_offsets_reading_of_ill_formed_prefixes():
    """An offset below its predecessor ends an empty group; offsets past total_M are
    cut there; rows past the last end belong to no group."""
    owner = oracle.offsets_row_groups(np.array([3, 1, 6, 20], np.int32), 8)
    assert owner.tolist() == [0, 0, 0, 2, 2, 2, 3, 3]
    owner = oracle.offsets_row_groups(np.array([-2, 2], np.int32), 5)
    assert owner.tolist() == [1, 1, -1, -1, -1]


def test_offsets_equals_stacked_with_differenced_sizes():
    sizes = np.array([5, 0, 9, 1, 7])
    XQ, WQ, xs, ws, _ = _rand_problem(34, sizes, 6, 64, 25)
    offs = np.cumsum(sizes).astype(np.int32)
    a = oracle.grouped_offsets(XQ, WQ, xs, ws, offs)
    b = oracle.grouped_stacked(XQ, WQ, xs, ws, sizes)
    assert np.array_equal(a.bits, b.bits) and np.array_equal(a.row_class, b.row_class)


def _check_batched(seed, G, M, N, K):
    XQ, WQ, xs, ws, _ = _rand_problem(seed, [M] * G, N, K)
    res = oracle.grouped_batched(XQ.reshape(G, M, K), WQ, xs.reshape(G, M), ws)
    return _rows_match_exact(res, exact_ref.stacked_exact(XQ, WQ, xs, ws, [M] * G))


@pytest.mark.parametrize("seed,G,M,N,K", [(41, 3, 2, 4, 48), (42, 1, 5, 3, 32)])
def test_batched_equals_exact_bruteforce(seed, G, M, N, K):
    assert _check_batched(seed, G, M, N, K)


def test_batched_single_group_is_a_plain_scaled_gemm():
    """G = 1: the batched layout is one GEMM, (dec(X) @ dec(W)^T) scaled by rows and
    columns, written here with numpy's matmul on float64 (exact at this size)."""
    rng = np.random.default_rng(43)
    XQ = rng.choice(FINITE_CODES, size=(1, 6, 96)).astype(np.uint8)
    WQ = rng.choice(FINITE_CODES, size=(1, 5, 96)).astype(np.uint8)
    xs = (2.0 ** rng.uniform(-4, 4, (1, 6))).astype(np.float32)
    ws = (2.0 ** rng.uniform(-4, 4, (1, 5))).astype(np.float32)
    x = torch.from_numpy(XQ[0]).view(torch.float8_e4m3fn).double().numpy()
    w = torch.from_numpy(WQ[0]).view(torch.float8_e4m3fn).double().numpy()
    ref = (x @ w.T) * xs[0].astype(np.float64)[:, None] * ws[0].astype(np.float64)[None, :]
    res = oracle.grouped_batched(XQ, WQ, xs, ws)
    assert np.array_equal(res.values[0], ref)
    assert np.all(res.row_class == oracle.ROW_WRITTEN)


def test_batched_k_zero_is_zero():
    res = oracle.grouped_batched(np.zeros((2, 3, 0), np.uint8), np.zeros((2, 4, 0), np.uint8),
                                 np.ones((2, 3), np.float32), np.ones((2, 4), np.float32))
    assert np.all(res.bits == 0) and np.all(res.row_class == oracle.ROW_ZEROED)


# ---------------------------------------------------------------------------
# n_offsets (3D-2D) and k_offsets (2D-2D) layouts
# ---------------------------------------------------------------------------

def _bits_match_exact(got_bits, exact):
    """bf16 bits against exact ones (None entries must be the untouched sentinel;
    either sign of zero accepted)."""
    got = np.asarray(got_bits).astype(np.int64).reshape(-1)
    flat = [x for row in np.asarray(exact, dtype=object).reshape(-1).tolist() for x in [row]]
    for gv, want in zip(got.tolist(), flat):
        if want is None:
            if gv != int(og.UNTOUCHED_SENTINEL):
                return False
        elif (want & 0x7FFF) == 0:
            if (gv & 0x7FFF) != 0:
                return False
        elif gv != want:
            return False
    return True


def _n_problem(seed, G, M, total_N, K):
    rng = np.random.default_rng(seed)
    XQ = rng.choice(FINITE_CODES, size=(G, M, K)).astype(np.uint8)
    WQ = rng.choice(FINITE_CODES, size=(total_N, K)).astype(np.uint8)
    xs = (2.0 ** rng.uniform(-12, 4, (G, M))).astype(np.float32)
    ws = (2.0 ** rng.uniform(-12, 4, total_N)).astype(np.float32)
    return XQ, WQ, xs, ws


def _k_problem(seed, G, M, N, total_K):
    rng = np.random.default_rng(seed)
    XQ = rng.choice(FINITE_CODES, size=(M, total_K)).astype(np.uint8)
    WQ = rng.choice(FINITE_CODES, size=(N, total_K)).astype(np.uint8)
    xs = (2.0 ** rng.uniform(-12, 4, (G, M))).astype(np.float32)
    ws = (2.0 ** rng.uniform(-12, 4, (G, N))).astype(np.float32)
    return XQ, WQ, xs, ws


# (seed, n_offsets, M, K, total_N): an empty group, odd widths, unowned trailing columns
N_OFFSETS_CASES = [
    (51, [3, 3, 8], 2, 48, 8),
    (52, [1, 6], 3, 32, 9),
    (53, [5], 2, 16, 5),
]


def _check_n_offsets(seed, offs, M, K, total_N):
    XQ, WQ, xs, ws = _n_problem(seed, len(offs), M, total_N, K)
    res = oracle.grouped_n_offsets(XQ, WQ, xs, ws, np.array(offs, np.int32))
    ok = _bits_match_exact(res.bits, exact_ref.n_offsets_exact(XQ, WQ, xs, ws, offs))
    owner = np.full(total_N, -1)
    prev = 0
    for g, o in enumerate(offs):
        owner[prev:o] = g
        prev = o
    want_cls = np.where(owner >= 0, oracle.ROW_WRITTEN, oracle.ROW_UNTOUCHED)
    return ok and np.array_equal(res.col_class, want_cls)


@pytest.mark.parametrize("seed,offs,M,K,total_N", N_OFFSETS_CASES)
def test_n_offsets_equals_exact_bruteforce(seed, offs, M, K, total_N):
    assert _check_n_offsets(seed, offs, M, K, total_N)


# (seed, k_offsets, M, N, total_K): an empty slice, unequal slices, a trailing unread part
K_OFFSETS_CASES = [
    (61, [16, 16, 48], 2, 3, 48),
    (62, [32, 48], 3, 2, 64),
    (63, [16], 2, 2, 16),
]


def _check_k_offsets(seed, offs, M, N, total_K):
    XQ, WQ, xs, ws = _k_problem(seed, len(offs), M, N, total_K)
    res = oracle.grouped_k_offsets(XQ, WQ, xs, ws, np.array(offs, np.int32))
    return _bits_match_exact(res.bits, exact_ref.k_offsets_exact(XQ, WQ, xs, ws, offs)) and \
        np.all(res.row_class == oracle.ROW_WRITTEN)


@pytest.mark.parametrize("seed,offs,M,N,total_K", K_OFFSETS_CASES)
def test_k_offsets_equals_exact_bruteforce(seed, offs, M, N, total_K):
    assert _check_k_offsets(seed, offs, M, N, total_K)


def test_n_and_k_offsets_reading_of_ill_formed_prefixes():
    owner = oracle.n_offsets_col_groups(np.array([4, 2, 7, 30], np.int32), 9)
    assert owner.tolist() == [0, 0, 0, 0, 2, 2, 2, 3, 3]
    assert oracle.k_offsets_slices(np.array([32, 16, 64, 999], np.int32), 80) == \
        [(0, 32), (32, 32), (32, 64), (64, 80)]
    assert oracle.k_offsets_slices(np.array([-16, 16], np.int32), 32) == [(0, 0), (0, 16)]


def test_n_offsets_single_group_is_a_plain_scaled_gemm():
    """One group owning every column: a plain GEMM of the slab against W, written
    with numpy's matmul on torch-decoded operands (exact at this size)."""
    XQ, WQ, xs, ws = _n_problem(54, 1, 5, 7, 96)
    x = torch.from_numpy(XQ[0]).view(torch.float8_e4m3fn).double().numpy()
    w = torch.from_numpy(WQ).view(torch.float8_e4m3fn).double().numpy()
    ref = (x @ w.T) * xs[0].astype(np.float64)[:, None] * ws.astype(np.float64)[None, :]
    res = oracle.grouped_n_offsets(XQ, WQ, xs, ws, np.array([7], np.int32))
    assert np.array_equal(res.values, ref)


def test_n_offsets_equal_widths_equals_batched():
    """Groups of equal width N: column block g of the n_offsets result is the
    batched layout's slab g (W's rows regrouped as [G, N, K])."""
    G, M, N, K = 3, 4, 5, 64
    XQ, WQ, xs, ws = _n_problem(55, G, M, G * N, K)
    a = oracle.grouped_n_offsets(XQ, WQ, xs, ws, np.arange(1, G + 1, dtype=np.int32) * N)
    b = oracle.grouped_batched(XQ, WQ.reshape(G, N, K), xs, ws.reshape(G, N))
    for g in range(G):
        assert np.array_equal(a.bits[:, g * N:(g + 1) * N], b.bits[g])


def test_k_offsets_slices_sum_to_the_full_contraction():
    """With unit scales the unrounded per-group results of a partition of K add up
    to the full-K product of torch-decoded operands, exactly (every partial sum is
    exact in fp64)."""
    G, M, N, total_K = 4, 3, 5, 160
    XQ, WQ, _, _ = _k_problem(64, G, M, N, total_K)
    one_x = np.ones((G, M), np.float32)
    one_w = np.ones((G, N), np.float32)
    res = oracle.grouped_k_offsets(XQ, WQ, one_x, one_w, np.array([48, 48, 112, 160], np.int32))
    x = torch.from_numpy(XQ).view(torch.float8_e4m3fn).double().numpy()
    w = torch.from_numpy(WQ).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(res.values.sum(axis=0), x @ w.T)
    assert np.all(res.values[1] == 0)          # the empty slice


def test_k_offsets_concatenated_slabs_equal_batched():
    """Slabs laid side by side along K, each group slicing its own: group g's output
    is the batched layout's slab g."""
    G, M, N, K = 3, 4, 5, 48
    rng = np.random.default_rng(65)
    Xb = rng.choice(FINITE_CODES, size=(G, M, K)).astype(np.uint8)
    Wb = rng.choice(FINITE_CODES, size=(G, N, K)).astype(np.uint8)
    xs = (2.0 ** rng.uniform(-8, 4, (G, M))).astype(np.float32)
    ws = (2.0 ** rng.uniform(-8, 4, (G, N))).astype(np.float32)
    a = oracle.grouped_k_offsets(np.concatenate(list(Xb), axis=1), np.concatenate(list(Wb), axis=1), xs, ws,
                                 np.arange(1, G + 1, dtype=np.int32) * K)
    b = oracle.grouped_batched(Xb, Wb, xs, ws)
    assert np.array_equal(a.bits, b.bits)


def test_k_offsets_single_signed_neighbours():
    """Constant single-signed data outside a group's slice: a read past the slice
    would add terms of one sign and move the result far past any rounding."""
    M, N = 2, 3
    XQ = np.full((M, 96), 0x38, np.uint8)      # 1.0 everywhere
    WQ = np.full((N, 96), 0x38, np.uint8)
    res = oracle.grouped_k_offsets(XQ, WQ, np.ones((3, M), np.float32), np.ones((3, N), np.float32),
                                   np.array([16, 48, 96], np.int32))
    assert res.values[:, 0, 0].tolist() == [16.0, 32.0, 48.0]


def test_n_and_k_offsets_k_zero():
    a = oracle.grouped_n_offsets(np.zeros((2, 3, 0), np.uint8), np.zeros((5, 0), np.uint8),
                                 np.ones((2, 3), np.float32), np.ones(5, np.float32), np.array([2, 5], np.int32))
    assert np.all(a.bits == 0) and np.all(a.col_class == oracle.ROW_ZEROED)
    b = oracle.grouped_k_offsets(np.zeros((3, 0), np.uint8), np.zeros((4, 0), np.uint8),
                                 np.ones((2, 3), np.float32), np.ones((2, 4), np.float32), np.array([0, 0], np.int32))
    assert b.bits.shape == (2, 3, 4) and np.all(b.bits == 0)


def _load_worked():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    K = ex["K"]

    def vec(spec):
        v = np.zeros(K, np.uint8)
        if "all" in spec:
            v[:] = int(spec["all"], 16)
        else:
            for k, c in spec.items():
                v[int(k)] = int(c, 16)
        return v

    rows = {name: vec(spec) for name, spec in ex["rows"].items()}
    W = np.stack([np.stack([vec(ex["weights"]["g0n0"]), vec(ex["weights"]["g0n1"])]),
                  np.stack([vec(ex["weights"]["g1n0"]), vec(ex["weights"]["g1n1"])])])
    xsd = dict(ex["x_scale"])
    xsd["nan"] = float("nan")
    ws = np.array(ex["w_scale"], np.float32)
    return ex, rows, W, xsd, ws


def test_worked_example_stacked():
    ex, rows, W, xsd, ws = _load_worked()
    order = ex["stacked"]["row_order"]
    XQ = np.stack([rows[r] for r in order])
    xs = np.array([xsd[r] for r in order], np.float32)
    res = oracle.grouped_stacked(XQ, W, xs, ws, np.array(ex["stacked"]["M_sizes"]))
    for i, want in enumerate(ex["stacked"]["expected_bits"]):
        if want is None:
            assert res.row_class[i] == oracle.ROW_UNTOUCHED
        else:
            assert res.row_class[i] == oracle.ROW_WRITTEN
            assert [int(b, 16) for b in want] == res.bits[i].tolist()


def test_worked_example_padded():
    ex, rows, W, xsd, ws = _load_worked()
    slabs = ex["padded"]["slabs"]
    XQ = np.stack([np.stack([rows[r] for r in s]) for s in slabs])
    xs = np.array([[xsd[r] for r in s] for s in slabs], np.float32)
    res = oracle.grouped_dynamic(XQ, W, xs, ws, np.array(ex["padded"]["zero_start_index_M"]))
    want = np.array([[[int(b, 16) for b in r] for r in s] for s in ex["padded"]["expected_bits"]])
    assert np.array_equal(res.bits, want)
    assert res.row_class.tolist() == [oracle.ROW_WRITTEN, oracle.ROW_ZEROED,
                                      oracle.ROW_WRITTEN, oracle.ROW_WRITTEN]


# ---------------------------------------------------------------------------
# invariants and closed forms
# ---------------------------------------------------------------------------

def test_summation_order_independent():
    XQ, WQ, xs, ws, sizes = _rand_problem(21, [5, 0, 7], 9, 160)
    base = oracle.grouped_stacked(XQ, WQ, xs, ws, sizes)
    perm = np.random.default_rng(3).permutation(160)
    res = oracle.grouped_stacked(XQ[:, perm], WQ[:, :, perm], xs, ws, sizes)
    assert np.array_equal(base.bits, res.bits)


def test_zero_padded_k_is_bit_identical():
    XQ, WQ, xs, ws, sizes = _rand_problem(22, [4, 6], 8, 144)
    base = oracle.grouped_stacked(XQ, WQ, xs, ws, sizes)
    pad = 256 - 144
    XQp = np.concatenate([XQ, np.zeros((XQ.shape[0], pad), np.uint8)], 1)
    WQp = np.concatenate([WQ, np.zeros(WQ.shape[:2] + (pad,), np.uint8)], 2)
    res = oracle.grouped_stacked(XQp, WQp, xs, ws, sizes)
    assert np.array_equal(base.bits, res.bits)


def test_rowwise_factorisation_equals_dequantised_gemm():
    """Scales factor out of the reduction: the result equals a GEMM on the
    dequantised operands (dec(X) * x_scale) @ (dec(W) * w_scale)^T, to 1 ulp."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((40, 272)).astype(np.float32)
    w = rng.standard_normal((24, 272)).astype(np.float32)
    from workloads import quantize_rows
    XQ, xs = quantize_rows(x)
    WQ, ws = quantize_rows(w)
    res = oracle.grouped_stacked(XQ, WQ[None], xs, ws[None], np.array([40]))
    torch_dec = lambda q: torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy()
    ref = (torch_dec(XQ) * xs[:, None].astype(np.float64)) @ (torch_dec(WQ) * ws[:, None].astype(np.float64)).T
    got = oracle.bf16_bits_to_f64(res.bits)
    assert np.all(np.abs(got - ref) <= oracle.bf16_ulp(ref))


def test_dynamic_equals_stacked_on_compacted_rows():
    rng = np.random.default_rng(24)
    G, em, N, K = 4, 9, 7, 64
    XQ = rng.choice(FINITE_CODES, size=(G, em, K)).astype(np.uint8)
    WQ = rng.choice(FINITE_CODES, size=(G, N, K)).astype(np.uint8)
    xs = (2.0 ** rng.uniform(-6, 2, (G, em))).astype(np.float32)
    ws = (2.0 ** rng.uniform(-6, 2, (G, N))).astype(np.float32)
    zsi = np.array([0, 9, 4, 1])
    dyn = oracle.grouped_dynamic(XQ, WQ, xs, ws, zsi)
    rows = np.concatenate([XQ[g, :zsi[g]] for g in range(G)])
    xsc = np.concatenate([xs[g, :zsi[g]] for g in range(G)])
    st = oracle.grouped_stacked(rows, WQ, xsc, ws, zsi)
    dyn_rows = np.concatenate([dyn.bits[g, :zsi[g]] for g in range(G)])
    assert np.array_equal(dyn_rows, st.bits)
    for g in range(G):
        assert np.all(dyn.bits[g, zsi[g]:] == 0)


def test_identity_weights_reproduce_a():
    """B = I (the diagnostic used for a lost accumulator slot): with W = 1.0 on the
    diagonal, w_scale = 1 and a power-of-two x_scale, Y = dec(XQ) * x_scale exactly."""
    rng = np.random.default_rng(25)
    K = 64
    XQ = rng.choice(FINITE_CODES, size=(12, K)).astype(np.uint8)
    WQ = np.zeros((1, K, K), np.uint8)
    WQ[0, np.arange(K), np.arange(K)] = 0x38
    xs = (2.0 ** rng.integers(-4, 4, 12)).astype(np.float32)
    res = oracle.grouped_stacked(XQ, WQ, xs, np.ones((1, K), np.float32), np.array([12]))
    tdec = torch.from_numpy(XQ).view(torch.float8_e4m3fn).float() * torch.from_numpy(xs)[:, None]
    want = tdec.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = res.bits.copy()
    zero = (want & 0x7FFF) == 0
    assert np.array_equal(got[~zero], want[~zero])
    assert np.all((got[zero] & 0x7FFF) == 0)


def test_one_hot_rows_closed_form():
    rng = np.random.default_rng(26)
    K, N = 48, 5
    for trial in range(20):
        a, b = rng.choice(FINITE_CODES, 2)
        k0 = rng.integers(K)
        XQ = np.zeros((1, K), np.uint8)
        XQ[0, k0] = a
        WQ = rng.choice(FINITE_CODES, size=(1, N, K)).astype(np.uint8)
        WQ[0, 2, k0] = b
        xs = np.float32([rng.uniform(0.1, 3)])
        ws = rng.uniform(0.1, 3, (1, N)).astype(np.float32)
        res = oracle.grouped_stacked(XQ, WQ, xs, ws, np.array([1]))
        from fractions import Fraction
        dec = exact_ref._DEC
        v = dec[a] * dec[WQ[0, 2, k0]] * Fraction(float(xs[0])) * Fraction(float(ws[0, 2]))
        want = exact_ref.bf16_bits_exact(v)
        if (want & 0x7FFF) == 0:
            assert (int(res.bits[0, 2]) & 0x7FFF) == 0
        else:
            assert int(res.bits[0, 2]) == want


def test_power_of_two_scale_doubles_exactly():
    XQ, WQ, xs, ws, sizes = _rand_problem(27, [3, 5], 6, 64)
    xs = np.clip(xs, 2.0 ** -8, None).astype(np.float32)
    a = oracle.grouped_stacked(XQ, WQ, xs, ws, sizes)
    b = oracle.grouped_stacked(XQ, WQ, (xs * 2).astype(np.float32), ws, sizes)
    assert np.array_equal(b.values, a.values * 2)


def test_row_classes_stacked():
    owner = oracle.stacked_row_groups(np.array([2, -1, 3]), 7)
    assert owner.tolist() == [0, 0, 2, 2, 2, -1, -1]
    owner = oracle.stacked_row_groups(np.array([2, 4, 3]), 5)
    assert owner.tolist() == [0, 0, 1, 1, 1]
    owner = oracle.stacked_row_groups(np.array([0, 0]), 3)
    assert owner.tolist() == [-1, -1, -1]


def test_row_classes_dynamic_and_zeroing_flag():
    c = oracle.dynamic_row_classes(np.array([0, 3, 9, -2]), 3, True)
    W, Z = oracle.ROW_WRITTEN, oracle.ROW_ZEROED
    assert c.tolist() == [[Z, Z, Z], [W, W, W], [W, W, W], [Z, Z, Z]]
    c = oracle.dynamic_row_classes(np.array([1]), 3, False)
    assert c.tolist() == [[W, oracle.ROW_UNTOUCHED, oracle.ROW_UNTOUCHED]]


def test_k_zero_returns_zeros_in_both_layouts():
    st = oracle.grouped_stacked(np.zeros((5, 0), np.uint8), np.zeros((2, 4, 0), np.uint8),
                                np.ones(5, np.float32), np.ones((2, 4), np.float32), np.array([2, 1]))
    assert np.all(st.bits == 0) and np.all(st.row_class == oracle.ROW_ZEROED)
    dy = oracle.grouped_dynamic(np.zeros((2, 3, 0), np.uint8), np.zeros((2, 4, 0), np.uint8),
                                np.ones((2, 3), np.float32), np.ones((2, 4), np.float32), np.array([1, 3]),
                                zeroing_output_tensor=False)
    assert np.all(dy.bits == 0) and np.all(dy.row_class == oracle.ROW_ZEROED)


def test_empty_and_full_groups():
    """An empty group produces no rows; a full group equals G = 1 on its slice."""
    XQ, WQ, xs, ws, sizes = _rand_problem(28, [0, 6, 0, 4], 7, 96)
    res = oracle.grouped_stacked(XQ, WQ, xs, ws, sizes)
    one = oracle.grouped_stacked(XQ[6:10], WQ[3:4], xs[6:10], ws[3:4], np.array([4]))
    assert np.array_equal(res.bits[6:10], one.bits)


def test_entries_match_full_result():
    XQ, WQ, xs, ws, sizes = _rand_problem(29, [3, 0, 5, 2], 11, 64, total_M=12)
    full = oracle.grouped_stacked(XQ, WQ, xs, ws, sizes)
    rows = np.array([0, 2, 3, 7, 9, 10, 11])
    cols = np.array([0, 5, 10])
    vals, bits, owner = oracle.stacked_entries(XQ, WQ, xs, ws, sizes, rows, cols)
    assert np.array_equal(bits, full.bits[np.ix_(rows, cols)])
    G, em = 3, 4
    rng = np.random.default_rng(30)
    XQd = rng.choice(FINITE_CODES, size=(G, em, 32)).astype(np.uint8)
    WQd = rng.choice(FINITE_CODES, size=(G, 6, 32)).astype(np.uint8)
    xsd = rng.uniform(0.5, 2, (G, em)).astype(np.float32)
    wsd = rng.uniform(0.5, 2, (G, 6)).astype(np.float32)
    zsi = np.array([2, 0, 4])
    fulld = oracle.grouped_dynamic(XQd, WQd, xsd, wsd, zsi)
    g = np.array([0, 0, 1, 2, 2])
    r = np.array([1, 3, 0, 2, 3])
    vals, bits, cls = oracle.dynamic_entries(XQd, WQd, xsd, wsd, zsi, g, r, np.arange(6))
    assert np.array_equal(bits, fulld.bits[g, r])


# ---------------------------------------------------------------------------
# planted mistakes: each must trip at least one pin
# ---------------------------------------------------------------------------

def _pins_pass():
    ok = all(_check_bruteforce(*c) for c in BRUTE_CASES)
    ok = ok and all(_check_offsets(*c) for c in OFFSETS_CASES)
    ok = ok and _check_batched(41, 3, 2, 4, 48)
    ok = ok and all(_check_n_offsets(*c) for c in N_OFFSETS_CASES)
    ok = ok and all(_check_k_offsets(*c) for c in K_OFFSETS_CASES)
    try:
        test_worked_example_stacked()
        test_worked_example_padded()
    except AssertionError:
        ok = False
    return ok


def _mut_transposed_index(a_codes, b_codes):
    return og.decode_e4m3fn(a_codes) @ og.decode_e4m3fn(b_codes[::-1]).T


def _mut_dropped_term(a_codes, b_codes):
    return og.decode_e4m3fn(a_codes[:, 1:]) @ og.decode_e4m3fn(b_codes[:, 1:]).T


def _mut_no_xscale(acc, xs, ws):
    return acc * np.asarray(ws, np.float64)[None, :]


def _mut_group_shift(M_sizes, total_M):
    return og.__dict__["_orig_rows"](np.roll(np.asarray(M_sizes), 1), total_M)


def _mut_offsets_start(offsets, total_M):
    """Reads offsets[g] as the start of group g instead of its end."""
    owner = np.full(int(total_M), -1, dtype=np.int64)
    o = np.asarray(offsets, np.int64).tolist() + [total_M]
    for g in range(len(o) - 1):
        owner[min(o[g], total_M):min(max(o[g + 1], o[g]), total_M)] = g
    return owner


def _mut_n_offsets_start(n_offsets, total_N):
    """Reads n_offsets[g] as the first column of group g instead of its end."""
    return _mut_offsets_start(n_offsets, total_N)


def _mut_k_slice_to_total(k_offsets, total_K):
    """Keys the end of every K slice on the total K instead of the group's own end."""
    out = []
    prev = 0
    for o in np.asarray(k_offsets, np.int64).tolist():
        end = min(max(o, prev), total_K)
        out.append((prev, total_K))
        prev = end
    return out


def _mut_k_slice_from_zero(k_offsets, total_K):
    """Starts every K slice at 0 (offsets read as slice lengths from the origin)."""
    out = []
    prev = 0
    for o in np.asarray(k_offsets, np.int64).tolist():
        end = min(max(o, prev), total_K)
        out.append((0, end))
        prev = end
    return out


def _mut_sign(codes):
    return np.abs(og._E4M3FN_TABLE[np.asarray(codes, np.uint8)])


def _mut_fp32_detour(v):
    x = torch.from_numpy(np.asarray(v, np.float64).astype(np.float32))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _mut_truncate(v):
    f = np.asarray(v, np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


@pytest.mark.parametrize("name,attr,fn", [
    ("transposed/reversed W index", "_accumulate", _mut_transposed_index),
    ("dropped K term", "_accumulate", _mut_dropped_term),
    ("x_scale dropped", "_apply_scales", _mut_no_xscale),
    ("wrong group", "stacked_row_groups", _mut_group_shift),
    ("offsets read as group starts", "offsets_row_groups", _mut_offsets_start),
    ("n_offsets read as group starts", "n_offsets_col_groups", _mut_n_offsets_start),
    ("K slice read to the total K", "k_offsets_slices", _mut_k_slice_to_total),
    ("K slice read from the origin", "k_offsets_slices", _mut_k_slice_from_zero),
    ("sign lost in decode", "decode_e4m3fn", _mut_sign),
    ("bf16 rounding truncates", "bf16_rne_from_f64", _mut_truncate),
])
def test_planted_mistake_is_caught(monkeypatch, name, attr, fn):
    assert _pins_pass()
    monkeypatch.setitem(og.__dict__, "_orig_rows", og.stacked_row_groups)
    monkeypatch.setattr(og, attr, fn)
    assert not _pins_pass(), f"planted mistake not caught: {name}"


def test_planted_double_rounding_is_caught(monkeypatch):
    monkeypatch.setattr(og, "bf16_rne_from_f64", _mut_fp32_detour)
    monkeypatch.setattr(oracle, "bf16_rne_from_f64", _mut_fp32_detour)
    with pytest.raises(AssertionError):
        test_bf16_golden_cases()


# ---------------------------------------------------------------------------
# rowwise activation quantisation (amax / 448 scales, e4m3fn RNE codes)
# ---------------------------------------------------------------------------

def _bf16_bits(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_e4m3fn_rne_matches_torch_cast():
    """The encoder against torch's own fp32 -> float8_e4m3fn cast (RNE) on random
    values, every code's value, and every midpoint between neighbouring codes."""
    rng = np.random.default_rng(50)
    pos = oracle.e4m3fn_table()[:0x7F]
    mids = (pos[1:] + pos[:-1]) / 2
    vals = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000),
                           2.0 ** rng.uniform(-12, -6, 2000), pos, -pos, mids, -mids,
                           np.nextafter(mids, 0), np.nextafter(mids, 1000)]).astype(np.float32)
    vals = vals[np.abs(vals) <= 448]
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3fn_rne(vals), want)


def test_quantize_closed_forms():
    # the largest magnitude of a row maps to +-448 (code 0x7E / 0xFE); zero rows get scale 1
    x = np.array([[3.0, -1.5, 0.25, 0.0], [0.0, 0.0, 0.0, 0.0], [-7.0, 7.0, 1.0, -0.0]], np.float32)
    q, s = oracle.quantize_rowwise(_bf16_bits(x))
    assert s[1] == 1.0 and np.all(q[1] == 0)
    assert s[0] == np.float32(3.0) / np.float32(448.0)
    assert q[0, 0] == 0x7E and q[2, 1] == 0x7E and q[2, 0] == 0xFE
    assert q[0, 3] == 0x00 and q[2, 3] == 0x80
    # a row of powers of two with amax 448 has scale 1 and exact codes
    p2 = np.array([[448.0, 1.0, -0.5, 2.0 ** -9]], np.float32)
    q2, s2 = oracle.quantize_rowwise(_bf16_bits(p2))
    assert s2[0] == 1.0
    assert np.array_equal(oracle.decode_e4m3fn(q2[0]), p2[0].astype(np.float64))


def test_quantize_error_within_half_a_code_step():
    rng = np.random.default_rng(51)
    x = rng.normal(0, 1, (64, 512)).astype(np.float32) * (2.0 ** rng.uniform(-8, 8, (64, 1))).astype(np.float32)
    bits = _bf16_bits(x)
    xb = oracle.bf16_bits_to_f64(bits)
    q, s = oracle.quantize_rowwise(bits)
    y = xb / s.astype(np.float64)[:, None]
    dec = oracle.decode_e4m3fn(q)
    pos = oracle.e4m3fn_table()[:0x7F]
    idx = np.clip(np.searchsorted(pos, np.abs(y)), 1, 0x7E)
    step = pos[idx] - pos[idx - 1]
    assert np.all(np.abs(dec - y) <= step / 2 * (1 + 1e-6))


def test_planted_truncation_in_quantiser_is_caught(monkeypatch):
    from oracle import quantize as oq

    def truncate(y):
        y = np.asarray(y, np.float32)
        a = np.abs(y).astype(np.float64)
        code = np.clip(np.searchsorted(oq._POS, a, side="right") - 1, 0, 0x7E).astype(np.uint8)
        return (code | np.where(np.signbit(y), np.uint8(0x80), np.uint8(0))).astype(np.uint8)

    monkeypatch.setattr(oq, "e4m3fn_rne", truncate)
    monkeypatch.setattr(oracle, "e4m3fn_rne", truncate)
    with pytest.raises(AssertionError):
        test_e4m3fn_rne_matches_torch_cast()


def _torch_quantize_rowwise(x_bits):
    """The amax/448 rowwise quantisation composed from torch's own CPU operations:
    fp32 amax and scale, torch's fp32 division, clamp to +-448, torch's cast to
    float8_e4m3fn."""
    x = torch.from_numpy(np.asarray(x_bits, np.uint16).view(np.int16).copy()).view(torch.bfloat16).float()
    amax = x.abs().amax(dim=1)
    s = amax / 448.0
    s = torch.where(amax == 0, torch.ones_like(s), s)
    y = torch.clamp(x / s[:, None], -448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), s.numpy()


def _quantize_pin_inputs():
    """About 1M bf16 values: N(0, 1) rows under scales 2^-8 .. 2^8, rows whose
    largest magnitude sits in the subnormal-scale range, a zero row, a single
    non-zero entry, signed zeros."""
    rng = np.random.default_rng(61)
    rows, K = 2048, 512
    x = rng.standard_normal((rows, K)).astype(np.float32)
    x *= (2.0 ** rng.uniform(-8, 8, (rows, 1))).astype(np.float32)
    x[0] = 0.0
    x[1] = 0.0
    x[1, 7] = -3.5
    x[2, ::2] = -0.0
    x[3] *= np.float32(2.0 ** -120)
    return _bf16_bits(x)


def test_quantize_rowwise_matches_torch_composition():
    """Codes and scales equal, bit for bit, a composition of torch's own fp32
    division, clamp and e4m3fn cast on ~1M values ([MSLK-471], Design notes: one
    scale per row, constant along K)."""
    bits = _quantize_pin_inputs()
    q, s = oracle.quantize_rowwise(bits)
    q_t, s_t = _torch_quantize_rowwise(bits)
    assert np.array_equal(s.view(np.uint32), s_t.view(np.uint32))
    assert np.array_equal(q, q_t)


def test_planted_reciprocal_quotient_is_caught(monkeypatch):
    """x * (1 / s) rounds twice and changes some codes: the torch composition pin
    catches it."""
    from oracle import quantize as oq

    def reciprocal(x, s):
        with np.errstate(over="ignore"):   # 1 / s overflows for the subnormal-scale row
            r = (np.float32(1.0) / np.asarray(s, np.float32)).astype(np.float32)
        return (np.asarray(x, np.float32) * r[:, None]).astype(np.float32)

    monkeypatch.setattr(oq, "row_quotient", reciprocal)
    with pytest.raises(AssertionError):
        test_quantize_rowwise_matches_torch_composition()
