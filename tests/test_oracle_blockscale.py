"""Pins for the block-scaled (groupwise) oracle, checked against things other than
itself: an exact rational brute force, the rowwise oracle where the two schemes
must agree, and planted mistakes that each must trip a pin."""
import numpy as np
import pytest

import oracle
from oracle import blockscale as ob
from tests import exact_ref

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _problem(seed, sizes, N, K, bk, bn, pow2=True):
    rng = np.random.default_rng(seed)
    sizes = np.asarray(sizes, np.int64)
    M = int(sizes.clip(0).sum())
    G = sizes.size
    XQ = rng.choice(FINITE, size=(M, K)).astype(np.uint8)
    WQ = rng.choice(FINITE, size=(G, N, K)).astype(np.uint8)
    if pow2:
        xs = (2.0 ** rng.integers(-8, 4, (M, K // bk))).astype(np.float32)
        ws = (2.0 ** rng.integers(-8, 4, (G, N // bn, K // bk))).astype(np.float32)
    else:
        xs = (2.0 ** rng.uniform(-8, 4, (M, K // bk))).astype(np.float32)
        ws = (2.0 ** rng.uniform(-8, 4, (G, N // bn, K // bk))).astype(np.float32)
    return XQ, WQ, xs, ws, sizes


# (seed, sizes, N, K, block_k, block_n, power-of-two scales)
CASES = [
    (1, [2, 0, 3], 8, 48, 16, 4, True),
    (2, [1, 2], 6, 32, 16, 2, False),
    (3, [3], 4, 64, 32, 4, False),
]


def _check(seed, sizes, N, K, bk, bn, pow2):
    XQ, WQ, xs, ws, sizes = _problem(seed, sizes, N, K, bk, bn, pow2)
    res = oracle.grouped_stacked_blockscale(XQ, WQ, xs, ws, sizes, bk, bn)
    exact = exact_ref.blockscale_exact(XQ, WQ, xs, ws, sizes, bk, bn)
    for r, row in enumerate(exact):
        if row is None:
            if res.row_class[r] != oracle.ROW_UNTOUCHED:
                return False
            continue
        got = res.bits[r].astype(np.int64)
        want = np.array(row, np.int64)
        zero = (want & 0x7FFF) == 0
        if not (np.array_equal(got[~zero], want[~zero]) and np.all((got[zero] & 0x7FFF) == 0)):
            return False
    return True


@pytest.mark.parametrize("case", CASES)
def test_blockscale_equals_exact_bruteforce(case):
    """Power-of-two scales make every fp64 step exact; with other scales the fp64
    sum of scaled partials is off by ~2^-52 relative, which moves no rounding here."""
    assert _check(*case)


def test_constant_block_scales_equal_the_rowwise_oracle():
    """Scales constant along K (power-of-two, so every step is exact): block scaling
    reduces to rowwise scaling with w_scale[g, n] = the block scale of column n."""
    bk, bn, N, K = 32, 4, 8, 96
    XQ, WQ, xs, ws, sizes = _problem(11, [3, 0, 4], N, K, bk, bn, True)
    xs = np.repeat(xs[:, :1], K // bk, axis=1)
    ws = np.repeat(ws[:, :, :1], K // bk, axis=2)
    a = oracle.grouped_stacked_blockscale(XQ, WQ, xs, ws, sizes, bk, bn)
    b = oracle.grouped_stacked(XQ, WQ, xs[:, 0], ws[:, np.arange(N) // bn, 0], sizes)
    assert np.array_equal(a.bits, b.bits) and np.array_equal(a.row_class, b.row_class)


def test_one_k_block_equals_the_rowwise_oracle_for_any_scales():
    bk, bn, N, K = 64, 2, 6, 64
    XQ, WQ, xs, ws, sizes = _problem(12, [2, 5], N, K, bk, bn, False)
    a = oracle.grouped_stacked_blockscale(XQ, WQ, xs, ws, sizes, bk, bn)
    b = oracle.grouped_stacked(XQ, WQ, xs[:, 0], ws[:, np.arange(N) // bn, 0], sizes)
    assert np.array_equal(a.bits, b.bits)


def test_blockscale_k_zero_is_zero():
    res = oracle.grouped_stacked_blockscale(np.zeros((3, 0), np.uint8), np.zeros((1, 4, 0), np.uint8),
                                            np.zeros((3, 0), np.float32), np.zeros((1, 1, 0), np.float32),
                                            np.array([3]), 128, 4)
    assert np.all(res.bits == 0) and np.all(res.row_class == oracle.ROW_ZEROED)


def _check_dynamic(seed, zsi, em, N, K, bk, bn, zeroing):
    """Padded layout against the exact brute force of the stacked layout on the
    compacted valid rows, and the row classes of the padding rows."""
    G = len(zsi)
    XQ, WQ, xs, ws, _ = _problem(seed, [em] * G, N, K, bk, bn, False)
    XQd, xsd = XQ.reshape(G, em, K), xs.reshape(G, em, K // bk)
    res = oracle.grouped_dynamic_blockscale(XQd, WQ, xsd, ws, zsi, zeroing, bk, bn)
    valid = np.clip(np.array(zsi), 0, em)
    rows = np.concatenate([g * em + np.arange(valid[g]) for g in range(G)]).astype(np.int64)
    exact = exact_ref.blockscale_exact(XQ[rows], WQ, xs[rows], ws, valid, bk, bn)
    got = res.bits.reshape(G * em, N)[rows]
    for r, row in enumerate(exact):
        want = np.array(row, np.int64)
        zero = (want & 0x7FFF) == 0
        g = got[r].astype(np.int64)
        if not (np.array_equal(g[~zero], want[~zero]) and np.all((g[zero] & 0x7FFF) == 0)):
            return False
    cls = res.row_class.reshape(G, em)
    pad = oracle.ROW_ZEROED if zeroing else oracle.ROW_UNTOUCHED
    for gi in range(G):
        if not (np.all(cls[gi, :valid[gi]] == oracle.ROW_WRITTEN) and np.all(cls[gi, valid[gi]:] == pad)):
            return False
    return True


@pytest.mark.parametrize("zeroing", [True, False])
def test_dynamic_blockscale_equals_exact_bruteforce_on_valid_rows(zeroing):
    assert _check_dynamic(21, [2, 0, 4, 9], 4, 6, 48, 16, 2, zeroing)


def test_dynamic_blockscale_padding_rows_are_zero_and_equal_stacked_on_compacted_rows():
    G, em, N, K, bk, bn = 3, 5, 8, 64, 32, 4
    XQ, WQ, xs, ws, _ = _problem(22, [em] * G, N, K, bk, bn, False)
    zsi = np.array([5, 0, 2])
    d = oracle.grouped_dynamic_blockscale(XQ.reshape(G, em, K), WQ, xs.reshape(G, em, K // bk), ws, zsi, True, bk, bn)
    rows = np.concatenate([g * em + np.arange(zsi[g]) for g in range(G)])
    st = oracle.grouped_stacked_blockscale(XQ[rows], WQ, xs[rows], ws, zsi, bk, bn)
    assert np.array_equal(d.bits.reshape(G * em, N)[rows], st.bits)
    pad = np.setdiff1d(np.arange(G * em), rows)
    assert np.all(d.bits.reshape(G * em, N)[pad] == 0)


def test_offsets_and_batched_blockscale_reduce_to_stacked():
    """The offsets layout with offsets = the running sum of M_sizes, and the batched
    layout with equal slabs, are the stacked layout on the same rows (the
    stacked block-scaled oracle is the one pinned to the exact brute force)."""
    bk, bn, N, K = 16, 4, 8, 48
    sizes = np.array([3, 0, 5, 2])
    XQ, WQ, xs, ws, _ = _problem(23, sizes, N, K, bk, bn, False)
    st = oracle.grouped_stacked_blockscale(XQ, WQ, xs, ws, sizes, bk, bn)
    of = oracle.grouped_offsets_blockscale(XQ, WQ, xs, ws, np.cumsum(sizes).astype(np.int32), bk, bn)
    assert np.array_equal(st.bits, of.bits) and np.array_equal(st.row_class, of.row_class)
    G, M = 3, 4
    XQ, WQ, xs, ws, _ = _problem(24, [M] * G, N, K, bk, bn, False)
    st = oracle.grouped_stacked_blockscale(XQ, WQ, xs, ws, [M] * G, bk, bn)
    ba = oracle.grouped_batched_blockscale(XQ.reshape(G, M, K), WQ, xs.reshape(G, M, -1), ws, bk, bn)
    assert np.array_equal(st.bits.reshape(G, M, N), ba.bits) and np.all(ba.row_class == oracle.ROW_WRITTEN)


def _pins_pass():
    return all(_check(*c) for c in CASES) and _check_dynamic(21, [2, 0, 4, 9], 4, 6, 48, 16, 2, True)


def _mut_shifted_scales(partials, xs, ws_cols):
    """The scales of block kb + 1 applied to block kb."""
    return ob.__dict__["_orig_scale"](partials, np.roll(xs, -1, axis=1), np.roll(ws_cols, -1, axis=1))


def _mut_block_boundary(a_codes, b_codes, block_k):
    """Blocks starting one element late (the last element of each block moves on)."""
    a = np.roll(a_codes, -1, axis=1)
    b = np.roll(b_codes, -1, axis=1)
    return ob.__dict__["_orig_partials"](a, b, block_k)


def _mut_column_block_modulo(N, block_n):
    return np.arange(N) % (N // block_n)


@pytest.mark.parametrize("name,attr,fn", [
    ("scales of the next K block", "scale_blocks", _mut_shifted_scales),
    ("K block boundaries off by one", "block_partials", _mut_block_boundary),
    ("column block taken modulo", "column_blocks", _mut_column_block_modulo),
])
def test_planted_mistake_is_caught(monkeypatch, name, attr, fn):
    assert _pins_pass()
    monkeypatch.setitem(ob.__dict__, "_orig_scale", ob.scale_blocks)
    monkeypatch.setitem(ob.__dict__, "_orig_partials", ob.block_partials)
    monkeypatch.setattr(ob, attr, fn)
    assert not _pins_pass(), f"planted mistake not caught: {name}"
