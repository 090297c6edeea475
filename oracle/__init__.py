"""CPU oracle for the FP8 rowwise-scaled grouped GEMM (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never does, and shares no code with it.
"""
from .grouped_gemm import (  # noqa: F401
    ROW_UNTOUCHED,
    ROW_WRITTEN,
    ROW_ZEROED,
    OracleResult,
    bf16_bits_to_f64,
    bf16_rne_from_f64,
    bf16_ulp,
    decode_e4m3fn,
    dynamic_entries,
    dynamic_row_classes,
    e4m3fn_table,
    k_offsets_slices,
    n_offsets_col_groups,
    grouped_batched,
    grouped_dynamic,
    grouped_k_offsets,
    grouped_n_offsets,
    grouped_offsets,
    grouped_stacked,
    offsets_row_groups,
    stacked_entries,
    stacked_row_groups,
)
from .quantize import e4m3fn_rne, quantize_rowwise  # noqa: F401,E402
from .blockscale import (grouped_batched_blockscale, grouped_dynamic_blockscale,  # noqa: F401,E402
                         grouped_offsets_blockscale, grouped_stacked_blockscale)
