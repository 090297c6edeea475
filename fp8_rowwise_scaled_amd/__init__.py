"""FP8 (e4m3fn) rowwise-scaled grouped GEMM for MI355X (gfx950).

The computation lives in the HIP library libfp8gg.so (C ABI: include/fp8gg.h);
this package holds its sources (csrc/), the build step and a thin binding.
"""
from ._lib import (  # noqa: F401
    LAYOUT_BATCHED,
    LAYOUT_K_OFFSETS,
    LAYOUT_N_OFFSETS,
    LAYOUT_OFFSETS,
    LAYOUT_PADDED,
    LAYOUT_STACKED,
    SHUFFLE_K,
    SHUFFLE_N,
    last_error,
    load,
    plan,
)
from .ops import (  # noqa: F401
    f8f8bf16_groupwise_grouped_batched,
    f8f8bf16_groupwise_grouped_batched_preshuffle,
    f8f8bf16_groupwise_grouped_dynamic,
    f8f8bf16_groupwise_grouped_dynamic_preshuffle,
    f8f8bf16_groupwise_grouped_offsets,
    f8f8bf16_groupwise_grouped_offsets_preshuffle,
    f8f8bf16_groupwise_grouped_stacked,
    f8f8bf16_groupwise_grouped_stacked_preshuffle,
    f8f8bf16_rowwise_grouped_batched,
    f8f8bf16_rowwise_grouped_batched_preshuffle,
    f8f8bf16_rowwise_grouped_dynamic,
    f8f8bf16_rowwise_grouped_dynamic_preshuffle,
    f8f8bf16_rowwise_grouped_k_offsets,
    f8f8bf16_rowwise_grouped_mm,
    f8f8bf16_rowwise_grouped_mm_preshuffle,
    f8f8bf16_rowwise_grouped_n_offsets,
    f8f8bf16_rowwise_grouped_offsets,
    f8f8bf16_rowwise_grouped_offsets_preshuffle,
    f8f8bf16_rowwise_grouped_stacked,
    f8f8bf16_quantize_rowwise,
    f8f8bf16_rowwise_grouped_stacked_preshuffle,
    f8f8bf16_shuffle_b,
)
