"""CPU-only checks of the C ABI: the library loads, exports every declared
symbol, plans launches, and refuses bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import fp8_rowwise_scaled_amd as F
from fp8_rowwise_scaled_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8gg.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(f8f8bf16_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert len(names) == 23
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_plan_gate_up():
    p = F.plan(F.LAYOUT_STACKED, False, 8, 4096, 4096, 7168)
    assert p["config_id"] >= 0 and p["k_tail"] == 0 and p["zero_fill"] == 0
    # upper bound of M tiles: ceil(total_M / BM) + G - 1, at most total_M
    assert p["m_tiles"] == min(-(-4096 // p["BM"]) + 7, 4096)
    assert p["n_tiles"] == -(-4096 // p["BN"])
    assert p["grid"] == p["m_tiles"] * p["n_tiles"]


def test_plan_offsets_matches_stacked():
    for args in [(8, 4096, 4096, 7168), (8, 2048, 7168, 2048), (8, 32, 7168, 2048), (16, 3, 512, 256)]:
        for pre in (False, True):
            assert F.plan(F.LAYOUT_OFFSETS, pre, *args) == F.plan(F.LAYOUT_STACKED, pre, *args)


def test_plan_batched_is_exact():
    G, M, N, K = 4, 512, 8192, 28672
    p = F.plan(F.LAYOUT_BATCHED, False, G, M, N, K)
    assert p["persistent"] == 1
    assert p["m_tiles"] == G * -(-M // p["BM"])
    assert p["grid"] == p["m_tiles"] * p["n_tiles"]
    q = F.plan(F.LAYOUT_BATCHED, False, 16, 40, 1024, 512)
    assert q["persistent"] == 0 and q["m_tiles"] == 16 * -(-40 // q["BM"])


def test_plan_refuses_unknown_layout():
    with pytest.raises(ValueError):
        F.plan(6, False, 1, 1, 8, 16)
    with pytest.raises(ValueError):
        F.plan(-1, False, 1, 1, 8, 16)


def test_plan_padded_tails():
    p = F.plan(F.LAYOUT_PADDED, False, 16, 512, 1000, 7184)
    assert p["k_tail"] == (7184 % p["BK"] != 0) == 1
    assert p["n_tail"] == (1000 % p["BN"] != 0)
    assert p["grid"] == p["m_tiles"] * p["n_tiles"] * 16


def test_plan_small_m_bound():
    p = F.plan(F.LAYOUT_STACKED, False, 8, 1, 7168, 2048)
    assert p["m_tiles"] == 1      # one row can fill at most one tile


def test_plan_empty_and_k_zero():
    assert F.plan(F.LAYOUT_STACKED, False, 8, 0, 64, 64)["config_id"] == -1
    assert F.plan(F.LAYOUT_STACKED, False, 8, 16, 0, 64)["config_id"] == -1
    p = F.plan(F.LAYOUT_PADDED, False, 2, 16, 64, 0)
    assert p["zero_fill"] == 1 and p["config_id"] == -1


@pytest.mark.parametrize("G,M,N,K", [(1, 4, 8, 24), (1, 4, 12, 32), (-1, 4, 8, 16), (1, -4, 8, 16)])
def test_plan_refuses_bad_shapes(G, M, N, K):
    with pytest.raises(ValueError):
        F.plan(F.LAYOUT_STACKED, False, G, M, N, K)


def test_preshuffle_granule_rule():
    with pytest.raises(ValueError):
        F.plan(F.LAYOUT_STACKED, True, 2, 64, 40, 128)   # N % 32
    with pytest.raises(ValueError):
        F.plan(F.LAYOUT_STACKED, True, 2, 64, 64, 80)    # K % 64


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_entry_points_refuse_before_any_gpu_call():
    lib = _lib.load()
    a = 0x10000000  # never dereferenced: every call below fails host-side checks
    # K % 16
    st = lib.f8f8bf16_rowwise_grouped_stacked(a, a, a, a, a, a + 0x1000000, 2, 8, 16, 24, None)
    assert st == _lib.ERR_UNSUPPORTED_SHAPE and "multiple of 16" in F.last_error()
    # null input
    st = lib.f8f8bf16_rowwise_grouped_stacked(None, a, a, a, a, a + 0x1000000, 2, 8, 16, 32, None)
    assert st == _lib.ERR_INVALID_ARGUMENT and "null" in F.last_error()
    # misaligned Y
    st = lib.f8f8bf16_rowwise_grouped_dynamic(a, a, a, a, a, a + 0x1000002, 2, 8, 16, 32, 1, None)
    assert st == _lib.ERR_INVALID_ARGUMENT and "aligned" in F.last_error()
    # Y overlapping XQ
    st = lib.f8f8bf16_rowwise_grouped_stacked(a, a + 0x100000, a + 0x200000, a + 0x300000, a + 0x400000,
                                              a + 0x10, 2, 8, 16, 32, None)
    assert st == _lib.ERR_INVALID_ARGUMENT and "overlaps" in F.last_error()
    # shuffle with overlap
    st = lib.f8f8bf16_shuffle_b(a, a + 64, 1, 32, 64, None)
    assert st == _lib.ERR_INVALID_ARGUMENT
    # empty output: nothing to do, even with null pointers
    st = lib.f8f8bf16_rowwise_grouped_stacked(None, None, None, None, None, None, 4, 0, 16, 32, None)
    assert st == _lib.OK and F.last_error() == ""


def test_last_error_is_per_thread():
    """Eight threads fail host-side checks concurrently, each with its own kind of
    error, and each reads back its own message (the message is thread-local; ctypes
    releases the GIL around every call, so the calls really overlap)."""
    import threading
    lib = _lib.load()
    a = 0x10000000
    calls = {
        "multiple of 16": lambda: lib.f8f8bf16_rowwise_grouped_stacked(a, a, a, a, a, a + 0x1000000, 2, 8, 16, 24,
                                                                       None),
        "null": lambda: lib.f8f8bf16_rowwise_grouped_stacked(None, a, a, a, a, a + 0x1000000, 2, 8, 16, 32, None),
        "aligned": lambda: lib.f8f8bf16_rowwise_grouped_dynamic(a, a, a, a, a, a + 0x1000002, 2, 8, 16, 32, 1,
                                                                None),
        "": lambda: lib.f8f8bf16_rowwise_grouped_stacked(None, None, None, None, None, None, 4, 0, 16, 32, None),
    }
    kinds = list(calls)
    failures = []
    start = threading.Barrier(8)

    def worker(t):
        start.wait()
        for i in range(300):
            kind = kinds[(t + i) % len(kinds)]
            calls[kind]()
            msg = F.last_error()
            if (kind == "" and msg != "") or kind not in msg:
                failures.append((t, i, kind, msg))
                return

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not failures, failures[:3]


def test_plan_n_offsets_bounds_column_tiles():
    """n_offsets: column tiles over the groups' ranges are at most ceil(N/BN) + G - 1
    (each holds a column), row tiles cover one slab."""
    for G, M, N, K in [(8, 512, 16384, 7168), (5, 40, 1000, 208), (64, 3, 64, 32)]:
        p = F.plan(F.LAYOUT_N_OFFSETS, False, G, M, N, K)
        assert p["n_tiles"] == min(-(-N // p["BN"]) + G - 1, N)
        assert p["m_tiles"] == -(-M // p["BM"])
        assert p["grid"] == p["m_tiles"] * p["n_tiles"]
        assert p["persistent"] == 0 and p["k_tail"] == (K % p["BK"] != 0)


def test_ragged_selector_takes_192_row_tiles_only_within_one_round():
    """Large ragged calls use 256x256 tiles, or 192x256 when those still make at most
    one round of 256 compute units (a host-side bound on the tile count)."""
    # 8 slabs of 512 rows, N = 16384: at most 3 x 71 = 213 tiles of 192x256
    p = F.plan(F.LAYOUT_N_OFFSETS, False, 8, 512, 16384, 7168)
    assert (p["BM"], p["BN"]) == (192, 256) and p["m_tiles"] * p["n_tiles"] <= 256
    # 2048-row slabs: 11 x 71 tiles would take several rounds
    p = F.plan(F.LAYOUT_N_OFFSETS, False, 8, 2048, 16384, 7168)
    assert (p["BM"], p["BN"]) == (256, 256)
    # k_offsets, the weight-gradient shape: 8 x 8 x 28 tiles of 256x256
    p = F.plan(F.LAYOUT_K_OFFSETS, False, 8, 2048, 7168, 4096)
    assert (p["BM"], p["BN"]) == (256, 256)
    # a small k_offsets call that fits one round either way
    p = F.plan(F.LAYOUT_K_OFFSETS, False, 2, 512, 1024, 4096)
    assert (p["BM"], p["BN"]) == (192, 256) and p["grid"] == 2 * 3 * 4


def test_plan_k_offsets_always_masks_the_tail():
    p = F.plan(F.LAYOUT_K_OFFSETS, False, 8, 2048, 7168, 4096)
    assert p["k_tail"] == 1 and p["persistent"] == 0
    assert p["grid"] == 8 * p["m_tiles"] * p["n_tiles"]


def test_ragged_layouts_refuse_preshuffled_weights():
    for layout in (F.LAYOUT_N_OFFSETS, F.LAYOUT_K_OFFSETS):
        with pytest.raises(ValueError, match="plain weights only"):
            F.plan(layout, True, 2, 64, 256, 256)


def test_ragged_layouts_refuse_configurations_not_built_for_them(monkeypatch):
    monkeypatch.setenv("FP8GG_CONFIG", "0")
    with pytest.raises(ValueError, match="not built"):
        F.plan(F.LAYOUT_N_OFFSETS, False, 2, 64, 256, 256)
    monkeypatch.setenv("FP8GG_CONFIG", "16")     # persistent: runs its one-tile twin
    assert F.plan(F.LAYOUT_K_OFFSETS, False, 2, 64, 256, 256)["config_id"] == 7


def test_ragged_entry_points_refuse_on_the_host():
    lib = _lib.load()
    a = 0x10000000
    st = lib.f8f8bf16_rowwise_grouped_n_offsets(a, a, a, a, a, a + 0x1000000, 2, 8, 12, 32, None)
    assert st == _lib.ERR_UNSUPPORTED_SHAPE and "multiple of 8" in F.last_error()
    # Y [G, M, N] = 2*8*16 bf16 = 512 bytes from a + 0x100: overlaps WQ at a + 0x200
    st = lib.f8f8bf16_rowwise_grouped_k_offsets(a + 0x10000, a + 0x200, a + 0x20000, a + 0x30000, a + 0x40000,
                                                a + 0x100, 2, 8, 16, 32, None)
    assert st == _lib.ERR_INVALID_ARGUMENT and "overlaps WQ" in F.last_error()
    st = lib.f8f8bf16_rowwise_grouped_k_offsets(a, a, a, a, a + 2, a + 0x1000000, 2, 8, 16, 32, None)
    assert st == _lib.ERR_INVALID_ARGUMENT and "aligned" in F.last_error()
    # no groups, no elements: nothing to do
    st = lib.f8f8bf16_rowwise_grouped_k_offsets(None, None, None, None, None, None, 0, 8, 16, 32, None)
    assert st == _lib.OK


def test_num_configs():
    assert _lib.load().f8f8bf16_num_configs() >= 1


def test_every_configuration_fits_lds(monkeypatch):
    """Each compiled configuration's LDS footprint fits a compute unit (160 KiB)."""
    for cfg in range(_lib.load().f8f8bf16_num_configs()):
        monkeypatch.setenv("FP8GG_CONFIG", str(cfg))
        try:                                  # a configuration serves plain or pre-shuffled W
            p = F.plan(F.LAYOUT_STACKED, False, 8, 4096, 4096, 7168)
        except ValueError:
            p = F.plan(F.LAYOUT_STACKED, True, 8, 4096, 4096, 7168)
        assert p["config_id"] == cfg
        assert 0 < p["lds_bytes"] <= 160 * 1024, (cfg, p["lds_bytes"])


@pytest.mark.parametrize("G,M,N,K", [
    (1 << 20, 1024, 1 << 20, 1 << 20),   # W would be 2^60 bytes
    (1, 1 << 30, 8, 1 << 20),            # X would be 2^50 bytes
    (1, 1 << 30, 1 << 20, 16),           # Y would be 2^51 bytes
])
def test_plan_refuses_tensors_past_2_to_48_bytes(G, M, N, K):
    with pytest.raises(ValueError, match="2\\^48"):
        F.plan(F.LAYOUT_STACKED, False, G, M, N, K)


def test_plan_accepts_large_but_sane_shapes():
    p = F.plan(F.LAYOUT_STACKED, False, 256, 1 << 20, 8192, 8192)   # W 16 GiB, X 8 GiB
    assert p["config_id"] >= 0


def test_quantize_refuses_bad_shapes_and_overlaps_on_the_host():
    """Checks run before any launch: fake device addresses never reach a kernel."""
    lib = _lib.load()
    base = 0x10000000
    # K not a multiple of 8
    assert lib.f8f8bf16_quantize_rowwise(base, base + (1 << 20), base + (2 << 20), 4, 12, None) == _lib.ERR_UNSUPPORTED_SHAPE
    # negative size
    assert lib.f8f8bf16_quantize_rowwise(base, base + (1 << 20), base + (2 << 20), -1, 8, None) == _lib.ERR_INVALID_ARGUMENT
    # XQ overlapping X
    assert lib.f8f8bf16_quantize_rowwise(base, base + 64, base + (2 << 20), 4, 64, None) == _lib.ERR_INVALID_ARGUMENT
    # misaligned X
    assert lib.f8f8bf16_quantize_rowwise(base + 8, base + (1 << 20), base + (2 << 20), 4, 64, None) == _lib.ERR_INVALID_ARGUMENT
    # null scale pointer
    assert lib.f8f8bf16_quantize_rowwise(base, base + (1 << 20), None, 4, 64, None) == _lib.ERR_INVALID_ARGUMENT
    # nothing to do: no launch, success
    assert lib.f8f8bf16_quantize_rowwise(None, None, None, 0, 64, None) == _lib.OK


def test_missing_library_raises(monkeypatch, tmp_path):
    """The product path has no fallback: without libfp8gg.so, loading raises."""
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libfp8gg.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.load()


def test_grouped_mm_needs_offsets_where_the_ranks_group_an_axis():
    import torch
    x2, w3 = torch.zeros((4, 32), dtype=torch.uint8), torch.zeros((2, 8, 32), dtype=torch.uint8)
    x3, w2 = torch.zeros((2, 4, 32), dtype=torch.uint8), torch.zeros((8, 32), dtype=torch.uint8)
    for a, b in ((x2, w3), (x3, w2), (x2, w2)):
        with pytest.raises(ValueError, match="offs"):
            F.f8f8bf16_rowwise_grouped_mm(a, b, None, None, None)
    with pytest.raises(ValueError, match="no grouped layout"):
        F.f8f8bf16_rowwise_grouped_mm(torch.zeros(4, dtype=torch.uint8), w3, None, None, torch.zeros(2))
