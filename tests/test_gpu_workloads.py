"""GPU parity at the full sizes of the five MoE-shaped workloads.

Each workload runs through the C ABI with the default configuration selector
(the launch that bench.py times).  The whole output is checked on the GPU for
row classification (no sentinel left in valid rows, zeros in padding rows, no
NaN); values are compared with the oracle on sampled rows (every group's first
and last rows plus random interior rows) over all or sampled columns.
"""
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


def sample_rows_stacked(sizes, total_M, seed, per_group=10):
    rng = np.random.default_rng(seed)
    rows, start = [], 0
    for s in np.clip(sizes, 0, None).tolist():
        if s:
            pick = {start, start + s - 1, start + min(s - 1, 1)}
            pick.update((start + rng.integers(0, s, min(per_group, s))).tolist())
            rows.extend(sorted(pick))
        start += s
    return np.array(sorted(set(r for r in rows if r < total_M)), np.int64)


def stacked_call(F, w, pre=False):
    whole, out = P.guarded_output((w.total_M, w.N))
    W = P.dev(w.WQ)
    if pre:
        W = F.f8f8bf16_shuffle_b(W)
        F.f8f8bf16_rowwise_grouped_stacked_preshuffle(P.dev(w.XQ), W, P.dev(w.x_scale), P.dev(w.w_scale),
                                                      P.dev(w.M_sizes), out=out)
    else:
        F.f8f8bf16_rowwise_grouped_stacked(P.dev(w.XQ), W, P.dev(w.x_scale), P.dev(w.w_scale),
                                           P.dev(w.M_sizes), out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    return out


def check_stacked_full_size(F, w, cols=None, pre=False, per_group=10, seed=0):
    print(f"case {w.name} pre={pre}", flush=True)
    out = stacked_call(F, w, pre)
    bits = out.view(torch.int16)
    R = int(min(np.clip(w.M_sizes, 0, None).sum(), w.total_M))
    # whole-output classification on the GPU
    assert int((bits[:R] == P.SENTINEL).sum()) == 0, "valid rows left unwritten"
    assert int(torch.isnan(out[:R].float()).sum()) == 0, "NaN in valid rows"
    if R < w.total_M:
        assert bool((bits[R:] == P.SENTINEL).all()), "rows past sum(M_sizes) were written"
    rows = sample_rows_stacked(w.M_sizes, w.total_M, seed, per_group)
    cols = np.arange(w.N) if cols is None else cols
    _, ref_bits, owner = oracle.stacked_entries(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes, rows, cols)
    got = P.bits_of(out)[np.ix_(rows, cols)]
    res = oracle.OracleResult(None, ref_bits, np.where(owner >= 0, oracle.ROW_WRITTEN, oracle.ROW_UNTOUCHED))
    P.assert_rows_match(got, res, label=w.name)
    return out


def test_gate_up_full_size_plain_and_preshuffled(F):
    """The bench workload through both entry points (the bench times the
    pre-shuffled one): every column of sampled rows against the oracle, and the two
    outputs equal bit for bit (same tiles, same K order)."""
    w = wl.moe_gate_up()
    plain = check_stacked_full_size(F, w, seed=1)
    pre = check_stacked_full_size(F, w, pre=True, seed=1)
    assert torch.equal(plain.view(torch.int16), pre.view(torch.int16)), "pre-shuffled differs from plain"


@pytest.mark.parametrize("total_M", wl.DOWN_PROJ_TOTAL_M)
def test_down_proj_full_size(F, total_M):
    w = wl.moe_down(total_M)
    if total_M <= 256:
        print(f"case {w.name} (whole output vs oracle)", flush=True)
        out = stacked_call(F, w)
        P.assert_rows_match(P.bits_of(out), oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes),
                            label=w.name)
    else:
        check_stacked_full_size(F, w, seed=total_M)


@pytest.fixture(scope="module")
def dense():
    return wl.dense_expert()


def test_dense_expert_full_size_plain_and_preshuffled(F, dense):
    cols = np.sort(np.random.default_rng(4).choice(dense.N, 384, replace=False))
    cols = np.unique(np.concatenate([cols, [0, 1, dense.N - 2, dense.N - 1]]))
    plain = check_stacked_full_size(F, dense, cols=cols, per_group=6, seed=4)
    pre = check_stacked_full_size(F, dense, cols=cols, pre=True, per_group=6, seed=4)
    assert torch.equal(plain.view(torch.int16), pre.view(torch.int16)), "pre-shuffled differs from plain"


def test_padded_tails_full_size(F):
    w = wl.padded_tails()
    print(f"case {w.name}", flush=True)
    whole, out = P.guarded_output((w.G, w.expected_m, w.N))
    F.f8f8bf16_rowwise_grouped_dynamic(P.dev(w.XQ), P.dev(w.WQ), P.dev(w.x_scale), P.dev(w.w_scale),
                                       P.dev(w.zero_start_index_M), zeroing_output_tensor=True, out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    bits = out.view(torch.int16)
    z = np.clip(w.zero_start_index_M, 0, w.expected_m)
    groups, rows = [], []
    rng = np.random.default_rng(5)
    for g in range(w.G):
        assert bool((bits[g, z[g]:] == 0).all()), f"padding rows of group {g} not zero"
        if z[g]:
            assert int((bits[g, :z[g]] == P.SENTINEL).sum()) == 0, f"valid rows of group {g} unwritten"
            assert int(torch.isnan(out[g, :z[g]].float()).sum()) == 0
            pick = sorted({0, int(z[g]) - 1, *rng.integers(0, z[g], 6).tolist()})
            groups += [g] * len(pick)
            rows += pick
    groups, rows = np.array(groups), np.array(rows)
    _, ref_bits, cls = oracle.dynamic_entries(w.XQ, w.WQ, w.x_scale, w.w_scale, w.zero_start_index_M,
                                              groups, rows, np.arange(w.N))
    got = P.bits_of(out)[groups, rows]
    P.assert_rows_match(got, oracle.OracleResult(None, ref_bits, cls), label=w.name)


def test_padded_tails_full_size_poisoned(F):
    """The padded-tails workload with everything the call must not read poisoned:
    padding rows of X hold NaN codes (0x7F) and NaN x_scale, and the empty group's
    weights and w_scale are NaN.  With zeroing on and off, the valid rows equal the
    clean call's bit for bit (same launch), padding rows are zero with zeroing on
    and keep the sentinel with zeroing off."""
    w = wl.padded_tails()
    z = np.clip(w.zero_start_index_M, 0, w.expected_m)
    assert (z == 0).any(), "the workload has an empty group"

    def call(XQ, WQ, xs, ws, zeroing):
        whole, out = P.guarded_output((w.G, w.expected_m, w.N))
        F.f8f8bf16_rowwise_grouped_dynamic(P.dev(XQ), P.dev(WQ), P.dev(xs), P.dev(ws),
                                           P.dev(w.zero_start_index_M), zeroing_output_tensor=zeroing, out=out)
        torch.cuda.synchronize()
        P.check_guards(whole)
        return out.view(torch.int16)

    XQ, xs, WQ, ws = w.XQ.copy(), w.x_scale.copy(), w.WQ.copy(), w.w_scale.copy()
    for g in range(w.G):
        XQ[g, z[g]:] = 0x7F
        xs[g, z[g]:] = np.nan
        if z[g] == 0:
            WQ[g] = 0x7F
            ws[g] = np.nan
    for zeroing in (True, False):
        print(f"case {w.name} poisoned zeroing={zeroing}", flush=True)
        clean = call(w.XQ, w.WQ, w.x_scale, w.w_scale, zeroing)
        bad = call(XQ, WQ, xs, ws, zeroing)
        for g in range(w.G):
            assert torch.equal(bad[g, :z[g]], clean[g, :z[g]]), f"group {g}: valid rows changed by the poison"
            pad = bad[g, z[g]:]
            if zeroing:
                assert bool((pad == 0).all()), f"group {g}: padding rows not zero"
            else:
                assert bool((pad == P.SENTINEL).all()), f"group {g}: padding rows written"


def test_tiny_full(F):
    w = wl.tiny_stacked()
    out = stacked_call(F, w)
    P.assert_rows_match(P.bits_of(out), oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes),
                        label=w.name)
