"""ctypes loader for libfp8gg.so (the C ABI declared in include/fp8gg.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8gg.so")

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_UNSUPPORTED_SHAPE = 2
ERR_HIP = 3

LAYOUT_STACKED = 0
LAYOUT_PADDED = 1
LAYOUT_OFFSETS = 2
LAYOUT_BATCHED = 3
LAYOUT_N_OFFSETS = 4
LAYOUT_K_OFFSETS = 5
SHUFFLE_N = 32
SHUFFLE_K = 64

# Every symbol include/fp8gg.h declares.
EXPORTS = (
    "f8f8bf16_rowwise_grouped_stacked",
    "f8f8bf16_rowwise_grouped_dynamic",
    "f8f8bf16_rowwise_grouped_stacked_preshuffle",
    "f8f8bf16_rowwise_grouped_dynamic_preshuffle",
    "f8f8bf16_rowwise_grouped_offsets",
    "f8f8bf16_rowwise_grouped_offsets_preshuffle",
    "f8f8bf16_rowwise_grouped_batched",
    "f8f8bf16_rowwise_grouped_batched_preshuffle",
    "f8f8bf16_rowwise_grouped_n_offsets",
    "f8f8bf16_rowwise_grouped_k_offsets",
    "f8f8bf16_groupwise_grouped_stacked",
    "f8f8bf16_groupwise_grouped_stacked_preshuffle",
    "f8f8bf16_groupwise_grouped_dynamic",
    "f8f8bf16_groupwise_grouped_offsets",
    "f8f8bf16_groupwise_grouped_offsets_preshuffle",
    "f8f8bf16_groupwise_grouped_batched",
    "f8f8bf16_groupwise_grouped_batched_preshuffle",
    "f8f8bf16_groupwise_grouped_dynamic_preshuffle",
    "f8f8bf16_shuffle_b",
    "f8f8bf16_quantize_rowwise",
    "f8f8bf16_last_error",
    "f8f8bf16_plan",
    "f8f8bf16_num_configs",
)


class Plan(ctypes.Structure):
    _fields_ = [
        ("config_id", ctypes.c_int32),
        ("BM", ctypes.c_int32),
        ("BN", ctypes.c_int32),
        ("BK", ctypes.c_int32),
        ("threads", ctypes.c_int32),
        ("stages", ctypes.c_int32),
        ("k_tail", ctypes.c_int32),
        ("n_tail", ctypes.c_int32),
        ("m_tiles", ctypes.c_int64),
        ("n_tiles", ctypes.c_int64),
        ("grid", ctypes.c_int64),
        ("zero_fill", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32),
        ("persistent", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def load() -> ctypes.CDLL:
    """Load libfp8gg.so from the package directory; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m fp8_rowwise_scaled_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    gemm = [P, P, P, P, P, P, I64, I64, I64, I64]
    lib.f8f8bf16_rowwise_grouped_stacked.argtypes = gemm + [P]
    lib.f8f8bf16_rowwise_grouped_stacked_preshuffle.argtypes = gemm + [P]
    lib.f8f8bf16_rowwise_grouped_dynamic.argtypes = gemm + [I, P]
    lib.f8f8bf16_rowwise_grouped_dynamic_preshuffle.argtypes = gemm + [I, P]
    lib.f8f8bf16_rowwise_grouped_offsets.argtypes = gemm + [P]
    lib.f8f8bf16_rowwise_grouped_offsets_preshuffle.argtypes = gemm + [P]
    lib.f8f8bf16_rowwise_grouped_n_offsets.argtypes = gemm + [P]
    lib.f8f8bf16_rowwise_grouped_k_offsets.argtypes = gemm + [P]
    lib.f8f8bf16_groupwise_grouped_stacked.argtypes = gemm + [P]
    lib.f8f8bf16_groupwise_grouped_stacked_preshuffle.argtypes = gemm + [P]
    lib.f8f8bf16_groupwise_grouped_dynamic.argtypes = gemm + [I, P]
    lib.f8f8bf16_groupwise_grouped_offsets.argtypes = gemm + [P]
    lib.f8f8bf16_groupwise_grouped_offsets_preshuffle.argtypes = gemm + [P]
    lib.f8f8bf16_groupwise_grouped_dynamic_preshuffle.argtypes = gemm + [I, P]
    batched = [P, P, P, P, P, I64, I64, I64, I64, P]
    lib.f8f8bf16_rowwise_grouped_batched.argtypes = batched
    lib.f8f8bf16_rowwise_grouped_batched_preshuffle.argtypes = batched
    lib.f8f8bf16_groupwise_grouped_batched.argtypes = batched
    lib.f8f8bf16_groupwise_grouped_batched_preshuffle.argtypes = batched
    for name in EXPORTS:
        if name.startswith(("f8f8bf16_rowwise_grouped_", "f8f8bf16_groupwise_grouped_")):
            getattr(lib, name).restype = I
    lib.f8f8bf16_shuffle_b.argtypes = [P, P, I64, I64, I64, P]
    lib.f8f8bf16_shuffle_b.restype = I
    lib.f8f8bf16_quantize_rowwise.argtypes = [P, P, P, I64, I64, P]
    lib.f8f8bf16_quantize_rowwise.restype = I
    lib.f8f8bf16_last_error.argtypes = []
    lib.f8f8bf16_last_error.restype = ctypes.c_char_p
    lib.f8f8bf16_plan.argtypes = [I, I, I64, I64, I64, I64, ctypes.POINTER(Plan)]
    lib.f8f8bf16_plan.restype = I
    lib.f8f8bf16_num_configs.argtypes = []
    lib.f8f8bf16_num_configs.restype = I32
    _lib = lib
    return lib


def last_error() -> str:
    return load().f8f8bf16_last_error().decode()


def check(status: int, what: str) -> None:
    if status == OK:
        return
    msg = f"{what}: {last_error()}"
    if status in (ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED_SHAPE):
        raise ValueError(msg)
    raise RuntimeError(msg)


def plan(layout: int, preshuffled: bool, G: int, M: int, N: int, K: int) -> dict:
    """Host-only launch plan for a call (no GPU needed)."""
    p = Plan()
    check(load().f8f8bf16_plan(layout, int(preshuffled), G, M, N, K, ctypes.byref(p)), "f8f8bf16_plan")
    return p.as_dict()
