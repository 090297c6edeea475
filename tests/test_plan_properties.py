"""Property-based checks of the host launch planner (CPU only).

For random shapes in every layout, f8f8bf16_plan must either refuse the call for
the documented reason or return a plan whose numbers the kernels can rely on: the
grid covers every tile any group split can produce (the device resolves groups
from metadata the host never reads), the tails are flagged exactly when the tile
does not divide the extent, the LDS footprint fits a compute unit, and only the
layouts that support them get persistent or ragged configurations.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import fp8_rowwise_scaled_amd as F

LAYOUTS = [F.LAYOUT_STACKED, F.LAYOUT_PADDED, F.LAYOUT_OFFSETS, F.LAYOUT_BATCHED, F.LAYOUT_N_OFFSETS,
           F.LAYOUT_K_OFFSETS]
RAGGED = (F.LAYOUT_N_OFFSETS, F.LAYOUT_K_OFFSETS)
PACKED = (F.LAYOUT_STACKED, F.LAYOUT_OFFSETS)
RAGGED_CONFIGS = {2, 7, 9, 18, 21, 28}
LDS_BYTES = 160 * 1024


def cdiv(a, b):
    return -(-a // b)


def split(total, parts, seed):
    """A random composition of `total` into `parts` non-negative parts."""
    if parts == 0:
        return []
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.integers(0, total + 1, parts - 1))
    return np.diff(np.concatenate([[0], cuts, [total]])).tolist()


shapes = st.fixed_dictionaries({
    "layout": st.sampled_from(LAYOUTS),
    "pre": st.booleans(),
    "G": st.integers(0, 300),
    "M": st.integers(0, 20000),
    "n8": st.integers(0, 2500),
    "k16": st.integers(0, 1300),
    "seed": st.integers(0, 2 ** 31 - 1),
})


@settings(max_examples=600, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(shapes)
def test_plan_invariants(s):
    layout, pre, G, M = s["layout"], s["pre"], s["G"], s["M"]
    N, K = 8 * s["n8"], 16 * s["k16"]
    if pre and layout in RAGGED:
        with pytest.raises(ValueError, match="plain weights only"):
            F.plan(layout, pre, G, M, N, K)
        return
    if pre and (N % 32 or K % 64):
        with pytest.raises(ValueError, match="pre-shuffled weights need"):
            F.plan(layout, pre, G, M, N, K)
        return
    p = F.plan(layout, pre, G, M, N, K)
    assert p == F.plan(layout, pre, G, M, N, K), "the plan is a function of the shape"
    rows = M if layout in PACKED or layout == F.LAYOUT_N_OFFSETS else G * M
    if rows == 0 or N == 0:
        assert p["config_id"] == -1 and p["zero_fill"] == 0
        return
    if K == 0:
        assert p["zero_fill"] == 1 and p["config_id"] == -1
        return
    if G == 0:
        assert p["config_id"] == -1
        return
    BM, BN, BK = p["BM"], p["BN"], p["BK"]
    assert p["config_id"] >= 0 and BM > 0 and BN > 0 and BK in (64, 128)
    assert 0 < p["lds_bytes"] <= LDS_BYTES
    assert p["threads"] in (128, 256, 512)
    assert p["n_tail"] == int(N % BN != 0)
    assert p["k_tail"] == (1 if layout == F.LAYOUT_K_OFFSETS else int(K % BK != 0))
    assert 0 < p["grid"] < 2 ** 31
    if layout in RAGGED:
        assert p["config_id"] in RAGGED_CONFIGS and p["persistent"] == 0
        if p["stages"] == 2:   # two X slots and three W slots (W copied two stages ahead)
            assert p["lds_bytes"] == (2 * BM + 3 * BN) * BK
    if layout == F.LAYOUT_PADDED:
        assert p["persistent"] == 0

    if layout in PACKED:
        assert p["n_tiles"] == cdiv(N, BN)
        assert p["m_tiles"] == min(cdiv(M, BM) + G - 1, M)
        assert p["grid"] == p["m_tiles"] * p["n_tiles"]
        # Any split of the rows over the groups fits the launched M tiles.
        sizes = split(M, G, s["seed"])
        assert sum(cdiv(m, BM) for m in sizes) <= p["m_tiles"]
    elif layout == F.LAYOUT_BATCHED:
        assert p["m_tiles"] == G * cdiv(M, BM) and p["n_tiles"] == cdiv(N, BN)
        assert p["grid"] == p["m_tiles"] * p["n_tiles"]
    elif layout == F.LAYOUT_PADDED:
        assert p["m_tiles"] == cdiv(M, BM) and p["n_tiles"] == cdiv(N, BN)
        assert p["grid"] == p["m_tiles"] * p["n_tiles"] * G
    elif layout == F.LAYOUT_N_OFFSETS:
        assert p["m_tiles"] == cdiv(M, BM)
        assert p["n_tiles"] == min(cdiv(N, BN) + G - 1, N)
        assert p["grid"] == p["m_tiles"] * p["n_tiles"]
        # Any split of W's rows over the groups fits the launched column tiles.
        widths = split(N, G, s["seed"])
        assert sum(cdiv(n, BN) for n in widths) <= p["n_tiles"]
    else:  # k_offsets
        assert p["m_tiles"] == cdiv(M, BM) and p["n_tiles"] == cdiv(N, BN)
        assert p["grid"] == p["m_tiles"] * p["n_tiles"] * G


@settings(max_examples=200, deadline=None)
@given(st.sampled_from(LAYOUTS), st.integers(1, 64), st.integers(1, 4096), st.integers(1, 500),
       st.integers(1, 500))
def test_plan_refuses_off_granule_shapes(layout, G, M, n, k):
    """N off the 8-column store granule or K off the 16-byte load granule is refused
    with the reason, in every layout."""
    if n % 8:
        with pytest.raises(ValueError, match="multiple of 8"):
            F.plan(layout, False, G, M, n, 16 * k)
    if k % 16:
        with pytest.raises(ValueError, match="multiple of 16"):
            F.plan(layout, False, G, M, 8 * n, k)
