"""Python entry points over the C ABI: argument marshalling only.

Every computation runs in the HIP kernels of libfp8gg.so; torch supplies device
memory and the current stream.  There is no CPU fallback: without the built
library these functions raise.
"""
from __future__ import annotations

import torch

from . import _lib

_FP8 = getattr(torch, "float8_e4m3fn", None)


def _bytes(t: torch.Tensor, name: str) -> torch.Tensor:
    dt = t.dtype
    if dt == torch.uint8:
        return t
    if _FP8 is not None and dt == _FP8:
        return t.view(torch.uint8)
    raise ValueError(f"{name} must be float8_e4m3fn or uint8 (raw e4m3fn bytes), got {dt}")


def _check(t: torch.Tensor, name: str, dtype, shape: tuple) -> None:
    # One combined test on the common path (a decode call is short enough that the
    # binding's own time shows); the separate tests below only name what failed.
    if t.dtype != dtype or t.shape != shape or not t.is_cuda or not t.is_contiguous():
        _refuse(t, name, dtype, shape)


def _refuse(t: torch.Tensor, name: str, dtype, shape: tuple) -> None:
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    raise ValueError(f"{name} must be contiguous")


def _on_gpu(t: torch.Tensor, name: str) -> None:
    """For XQ and WQ after _bytes (dtype settled) whose shape the caller has just
    read off the tensor itself: only placement and layout are left to check."""
    if not t.is_cuda or not t.is_contiguous():
        _refuse(t, name, t.dtype, tuple(t.shape))


# The current stream's raw handle without building a torch.cuda.Stream object per
# call (the same handle torch launches its own work on).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(dev: torch.device) -> int:
    if _raw_stream is not None:
        return _raw_stream(dev.index)
    return torch.cuda.current_stream(dev).cuda_stream


def _stacked(fn_name, XQ, WQ, x_scale, w_scale, M_sizes, out, meta_name="M_sizes", meta_dtype=torch.int64):
    XQ = _bytes(XQ, "XQ")
    WQ = _bytes(WQ, "WQ")
    if XQ.dim() != 2 or WQ.dim() != 3:
        raise ValueError("XQ must be [total_M, K] and WQ [G, N, K]")
    total_M, K = XQ.shape
    G, N, K2 = WQ.shape
    if K2 != K:
        raise ValueError(f"K mismatch: XQ has {K}, WQ has {K2}")
    _on_gpu(XQ, "XQ")
    _on_gpu(WQ, "WQ")
    _check(x_scale, "x_scale", torch.float32, (total_M,))
    _check(w_scale, "w_scale", torch.float32, (G, N))
    _check(M_sizes, meta_name, meta_dtype, (G,))
    if out is None:
        out = torch.empty((total_M, N), dtype=torch.bfloat16, device=XQ.device)
    _check(out, "out", torch.bfloat16, (total_M, N))
    lib = _lib.load()
    st = getattr(lib, fn_name)(XQ.data_ptr(), WQ.data_ptr(), x_scale.data_ptr(), w_scale.data_ptr(),
                               M_sizes.data_ptr(), out.data_ptr(), G, total_M, N, K, _stream(XQ.device))
    _lib.check(st, fn_name)
    return out


def _dynamic(fn_name, XQ, WQ, x_scale, w_scale, zero_start_index_M, zeroing_output_tensor, out):
    XQ = _bytes(XQ, "XQ")
    WQ = _bytes(WQ, "WQ")
    if XQ.dim() != 3 or WQ.dim() != 3:
        raise ValueError("XQ must be [G, expected_m, K] and WQ [G, N, K]")
    G, em, K = XQ.shape
    G2, N, K2 = WQ.shape
    if G2 != G or K2 != K:
        raise ValueError(f"shape mismatch: XQ {tuple(XQ.shape)} vs WQ {tuple(WQ.shape)}")
    _on_gpu(XQ, "XQ")
    _on_gpu(WQ, "WQ")
    _check(x_scale, "x_scale", torch.float32, (G, em))
    _check(w_scale, "w_scale", torch.float32, (G, N))
    _check(zero_start_index_M, "zero_start_index_M", torch.int64, (G,))
    if out is None:
        out = torch.empty((G, em, N), dtype=torch.bfloat16, device=XQ.device)
    _check(out, "out", torch.bfloat16, (G, em, N))
    lib = _lib.load()
    st = getattr(lib, fn_name)(XQ.data_ptr(), WQ.data_ptr(), x_scale.data_ptr(), w_scale.data_ptr(),
                               zero_start_index_M.data_ptr(), out.data_ptr(), G, em, N, K,
                               int(bool(zeroing_output_tensor)), _stream(XQ.device))
    _lib.check(st, fn_name)
    return out


def f8f8bf16_rowwise_grouped_stacked(XQ, WQ, x_scale, w_scale, M_sizes, out=None):
    """Y [total_M, N] bf16 for the stacked layout (see include/fp8gg.h)."""
    return _stacked("f8f8bf16_rowwise_grouped_stacked", XQ, WQ, x_scale, w_scale, M_sizes, out)


def f8f8bf16_rowwise_grouped_stacked_preshuffle(XQ, WQs, x_scale, w_scale, M_sizes, out=None):
    """As the stacked op, with WQs produced by f8f8bf16_shuffle_b."""
    return _stacked("f8f8bf16_rowwise_grouped_stacked_preshuffle", XQ, WQs, x_scale, w_scale, M_sizes, out)


def f8f8bf16_rowwise_grouped_dynamic(XQ, WQ, x_scale, w_scale, zero_start_index_M,
                                     zeroing_output_tensor=True, out=None):
    """Y [G, expected_m, N] bf16 for the padded layout (see include/fp8gg.h)."""
    return _dynamic("f8f8bf16_rowwise_grouped_dynamic", XQ, WQ, x_scale, w_scale, zero_start_index_M,
                    zeroing_output_tensor, out)


def f8f8bf16_rowwise_grouped_dynamic_preshuffle(XQ, WQs, x_scale, w_scale, zero_start_index_M,
                                                zeroing_output_tensor=True, out=None):
    """As the dynamic op, with WQs produced by f8f8bf16_shuffle_b."""
    return _dynamic("f8f8bf16_rowwise_grouped_dynamic_preshuffle", XQ, WQs, x_scale, w_scale,
                    zero_start_index_M, zeroing_output_tensor, out)


def _batched(fn_name, XQ, WQ, x_scale, w_scale, out):
    XQ = _bytes(XQ, "XQ")
    WQ = _bytes(WQ, "WQ")
    if XQ.dim() != 3 or WQ.dim() != 3:
        raise ValueError("XQ must be [G, M, K] and WQ [G, N, K]")
    G, M, K = XQ.shape
    G2, N, K2 = WQ.shape
    if G2 != G or K2 != K:
        raise ValueError(f"shape mismatch: XQ {tuple(XQ.shape)} vs WQ {tuple(WQ.shape)}")
    _on_gpu(XQ, "XQ")
    _on_gpu(WQ, "WQ")
    _check(x_scale, "x_scale", torch.float32, (G, M))
    _check(w_scale, "w_scale", torch.float32, (G, N))
    if out is None:
        out = torch.empty((G, M, N), dtype=torch.bfloat16, device=XQ.device)
    _check(out, "out", torch.bfloat16, (G, M, N))
    lib = _lib.load()
    st = getattr(lib, fn_name)(XQ.data_ptr(), WQ.data_ptr(), x_scale.data_ptr(), w_scale.data_ptr(),
                               out.data_ptr(), G, M, N, K, _stream(XQ.device))
    _lib.check(st, fn_name)
    return out


def f8f8bf16_rowwise_grouped_offsets(XQ, WQ, x_scale, w_scale, offsets, out=None):
    """Y [total_M, N] bf16 for the offsets layout: offsets [G] int32 inclusive
    prefix sums of the group row counts (see include/fp8gg.h)."""
    return _stacked("f8f8bf16_rowwise_grouped_offsets", XQ, WQ, x_scale, w_scale, offsets, out,
                    "offsets", torch.int32)


def f8f8bf16_rowwise_grouped_offsets_preshuffle(XQ, WQs, x_scale, w_scale, offsets, out=None):
    """As the offsets op, with WQs produced by f8f8bf16_shuffle_b."""
    return _stacked("f8f8bf16_rowwise_grouped_offsets_preshuffle", XQ, WQs, x_scale, w_scale, offsets, out,
                    "offsets", torch.int32)


def f8f8bf16_rowwise_grouped_batched(XQ, WQ, x_scale, w_scale, out=None):
    """Y [G, M, N] bf16 for the batched layout: every group a full slab of M rows
    (see include/fp8gg.h)."""
    return _batched("f8f8bf16_rowwise_grouped_batched", XQ, WQ, x_scale, w_scale, out)


def f8f8bf16_rowwise_grouped_batched_preshuffle(XQ, WQs, x_scale, w_scale, out=None):
    """As the batched op, with WQs produced by f8f8bf16_shuffle_b."""
    return _batched("f8f8bf16_rowwise_grouped_batched_preshuffle", XQ, WQs, x_scale, w_scale, out)


def f8f8bf16_rowwise_grouped_n_offsets(XQ, WQ, x_scale, w_scale, n_offsets, out=None):
    """Y [M, total_N] bf16 for the n_offsets (3D-2D) layout: XQ [G, M, K], WQ
    [total_N, K], x_scale [G, M], w_scale [total_N], n_offsets [G] int32 inclusive
    prefix over W's rows (see include/fp8gg.h)."""
    XQ = _bytes(XQ, "XQ")
    WQ = _bytes(WQ, "WQ")
    if XQ.dim() != 3 or WQ.dim() != 2:
        raise ValueError("XQ must be [G, M, K] and WQ [total_N, K]")
    G, M, K = XQ.shape
    N, K2 = WQ.shape
    if K2 != K:
        raise ValueError(f"K mismatch: XQ has {K}, WQ has {K2}")
    _on_gpu(XQ, "XQ")
    _on_gpu(WQ, "WQ")
    _check(x_scale, "x_scale", torch.float32, (G, M))
    _check(w_scale, "w_scale", torch.float32, (N,))
    _check(n_offsets, "n_offsets", torch.int32, (G,))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=XQ.device)
    _check(out, "out", torch.bfloat16, (M, N))
    st = _lib.load().f8f8bf16_rowwise_grouped_n_offsets(XQ.data_ptr(), WQ.data_ptr(), x_scale.data_ptr(),
                                                        w_scale.data_ptr(), n_offsets.data_ptr(), out.data_ptr(),
                                                        G, M, N, K, _stream(XQ.device))
    _lib.check(st, "f8f8bf16_rowwise_grouped_n_offsets")
    return out


def f8f8bf16_rowwise_grouped_k_offsets(XQ, WQ, x_scale, w_scale, k_offsets, out=None):
    """Y [G, M, N] bf16 for the k_offsets (2D-2D) layout: XQ [M, total_K], WQ
    [N, total_K], x_scale [G, M], w_scale [G, N], k_offsets [G] int32 inclusive
    prefix over K, multiples of 16 (see include/fp8gg.h)."""
    XQ = _bytes(XQ, "XQ")
    WQ = _bytes(WQ, "WQ")
    if XQ.dim() != 2 or WQ.dim() != 2:
        raise ValueError("XQ must be [M, total_K] and WQ [N, total_K]")
    M, K = XQ.shape
    N, K2 = WQ.shape
    if K2 != K:
        raise ValueError(f"K mismatch: XQ has {K}, WQ has {K2}")
    if k_offsets.dim() != 1:
        raise ValueError("k_offsets must be [G]")
    G = k_offsets.shape[0]
    _on_gpu(XQ, "XQ")
    _on_gpu(WQ, "WQ")
    _check(x_scale, "x_scale", torch.float32, (G, M))
    _check(w_scale, "w_scale", torch.float32, (G, N))
    _check(k_offsets, "k_offsets", torch.int32, (G,))
    if out is None:
        out = torch.empty((G, M, N), dtype=torch.bfloat16, device=XQ.device)
    _check(out, "out", torch.bfloat16, (G, M, N))
    st = _lib.load().f8f8bf16_rowwise_grouped_k_offsets(XQ.data_ptr(), WQ.data_ptr(), x_scale.data_ptr(),
                                                        w_scale.data_ptr(), k_offsets.data_ptr(), out.data_ptr(),
                                                        G, M, N, K, _stream(XQ.device))
    _lib.check(st, "f8f8bf16_rowwise_grouped_k_offsets")
    return out


def f8f8bf16_rowwise_grouped_mm(XQ, WQ, x_scale, w_scale, offs=None, out=None):
    """The grouped mm: picks the grouped axis from the operand ranks ([MSLK-471],
    commit mapping the four rank combinations onto the kernel's layouts):
    2D-3D -> offsets (groups along M), 3D-3D -> batched (offs unused),
    3D-2D -> n_offsets (groups along N), 2D-2D -> k_offsets (groups along K)."""
    ra, rb = XQ.dim(), WQ.dim()
    if offs is None and (ra, rb) != (3, 3):
        raise ValueError(f"operand ranks {ra}D-{rb}D group along an axis given by offs, which is missing")
    if (ra, rb) == (2, 3):
        return f8f8bf16_rowwise_grouped_offsets(XQ, WQ, x_scale, w_scale, offs, out=out)
    if (ra, rb) == (3, 3):
        return f8f8bf16_rowwise_grouped_batched(XQ, WQ, x_scale, w_scale, out=out)
    if (ra, rb) == (3, 2):
        return f8f8bf16_rowwise_grouped_n_offsets(XQ, WQ, x_scale, w_scale, offs, out=out)
    if (ra, rb) == (2, 2):
        return f8f8bf16_rowwise_grouped_k_offsets(XQ, WQ, x_scale, w_scale, offs, out=out)
    raise ValueError(f"no grouped layout for operand ranks {ra}D-{rb}D")


def f8f8bf16_rowwise_grouped_mm_preshuffle(XQ, WQs, x_scale, w_scale, offs=None, out=None):
    """The grouped mm on pre-shuffled weights: only the ranks where every group
    owns a whole [N, K] (2D-3D, 3D-3D); the others raise rather than read shuffled
    weights as plain ones."""
    ra, rb = XQ.dim(), WQs.dim()
    if offs is None and (ra, rb) == (2, 3):
        raise ValueError("operand ranks 2D-3D group along M by offs, which is missing")
    if (ra, rb) == (2, 3):
        return f8f8bf16_rowwise_grouped_offsets_preshuffle(XQ, WQs, x_scale, w_scale, offs, out=out)
    if (ra, rb) == (3, 3):
        return f8f8bf16_rowwise_grouped_batched_preshuffle(XQ, WQs, x_scale, w_scale, out=out)
    raise ValueError(f"pre-shuffled weights are not accepted for operand ranks {ra}D-{rb}D "
                     "(the groups would split the shuffled blocks)")


def f8f8bf16_groupwise_grouped_stacked(XQ, WQ, x_scale, w_scale, M_sizes, out=None):
    """Y [total_M, N] bf16 for the stacked layout with block scales: x_scale
    [total_M, K/128], w_scale [G, N/128, K/128] (see include/fp8gg.h)."""
    return _groupwise("f8f8bf16_groupwise_grouped_stacked", XQ, WQ, x_scale, w_scale, M_sizes, out)


def f8f8bf16_groupwise_grouped_stacked_preshuffle(XQ, WQs, x_scale, w_scale, M_sizes, out=None):
    """As the block-scaled stacked op, with WQs produced by f8f8bf16_shuffle_b."""
    return _groupwise("f8f8bf16_groupwise_grouped_stacked_preshuffle", XQ, WQs, x_scale, w_scale, M_sizes, out)


def f8f8bf16_groupwise_grouped_dynamic(XQ, WQ, x_scale, w_scale, zero_start_index_M, zeroing_output_tensor=True,
                                       out=None):
    """Y [G, expected_m, N] bf16 for the padded layout with block scales: x_scale
    [G, expected_m, K/128], w_scale [G, N/128, K/128] (see include/fp8gg.h)."""
    return _groupwise_dynamic("f8f8bf16_groupwise_grouped_dynamic", XQ, WQ, x_scale, w_scale, zero_start_index_M,
                              zeroing_output_tensor, out)


def f8f8bf16_groupwise_grouped_dynamic_preshuffle(XQ, WQs, x_scale, w_scale, zero_start_index_M,
                                                  zeroing_output_tensor=True, out=None):
    """As the block-scaled padded op, with WQs produced by f8f8bf16_shuffle_b."""
    return _groupwise_dynamic("f8f8bf16_groupwise_grouped_dynamic_preshuffle", XQ, WQs, x_scale, w_scale,
                              zero_start_index_M, zeroing_output_tensor, out)


def _groupwise_dynamic(fn_name, XQ, WQ, x_scale, w_scale, zero_start_index_M, zeroing_output_tensor, out):
    XQ = _bytes(XQ, "XQ")
    WQ = _bytes(WQ, "WQ")
    if XQ.dim() != 3 or WQ.dim() != 3:
        raise ValueError("XQ must be [G, expected_m, K] and WQ [G, N, K]")
    G, em, K = XQ.shape
    G2, N, K2 = WQ.shape
    if G2 != G or K2 != K:
        raise ValueError(f"shape mismatch: XQ {tuple(XQ.shape)} vs WQ {tuple(WQ.shape)}")
    if K % 128 or N % 128:
        raise ValueError(f"block scaling needs K and N to be multiples of 128 (N={N}, K={K})")
    _on_gpu(XQ, "XQ")
    _on_gpu(WQ, "WQ")
    _check(x_scale, "x_scale", torch.float32, (G, em, K // 128))
    _check(w_scale, "w_scale", torch.float32, (G, N // 128, K // 128))
    _check(zero_start_index_M, "zero_start_index_M", torch.int64, (G,))
    if out is None:
        out = torch.empty((G, em, N), dtype=torch.bfloat16, device=XQ.device)
    _check(out, "out", torch.bfloat16, (G, em, N))
    st = getattr(_lib.load(), fn_name)(XQ.data_ptr(), WQ.data_ptr(), x_scale.data_ptr(), w_scale.data_ptr(),
                                       zero_start_index_M.data_ptr(), out.data_ptr(), G, em, N, K,
                                       int(bool(zeroing_output_tensor)), _stream(XQ.device))
    _lib.check(st, fn_name)
    return out


def f8f8bf16_groupwise_grouped_offsets(XQ, WQ, x_scale, w_scale, offsets, out=None):
    """Y [total_M, N] bf16 for the offsets layout (int32 inclusive prefix) with
    block scales (see include/fp8gg.h)."""
    return _groupwise("f8f8bf16_groupwise_grouped_offsets", XQ, WQ, x_scale, w_scale, offsets, out,
                      "offsets", torch.int32)


def f8f8bf16_groupwise_grouped_offsets_preshuffle(XQ, WQs, x_scale, w_scale, offsets, out=None):
    """As the block-scaled offsets op, with WQs produced by f8f8bf16_shuffle_b."""
    return _groupwise("f8f8bf16_groupwise_grouped_offsets_preshuffle", XQ, WQs, x_scale, w_scale, offsets, out,
                      "offsets", torch.int32)


def f8f8bf16_groupwise_grouped_batched(XQ, WQ, x_scale, w_scale, out=None):
    """Y [G, M, N] bf16 for the batched layout with block scales: XQ [G, M, K],
    x_scale [G, M, K/128], w_scale [G, N/128, K/128] (see include/fp8gg.h)."""
    return _groupwise_batched("f8f8bf16_groupwise_grouped_batched", XQ, WQ, x_scale, w_scale, out)


def f8f8bf16_groupwise_grouped_batched_preshuffle(XQ, WQs, x_scale, w_scale, out=None):
    """As the block-scaled batched op, with WQs produced by f8f8bf16_shuffle_b."""
    return _groupwise_batched("f8f8bf16_groupwise_grouped_batched_preshuffle", XQ, WQs, x_scale, w_scale, out)


def _groupwise_batched(fn_name, XQ, WQ, x_scale, w_scale, out):
    XQ = _bytes(XQ, "XQ")
    WQ = _bytes(WQ, "WQ")
    if XQ.dim() != 3 or WQ.dim() != 3:
        raise ValueError("XQ must be [G, M, K] and WQ [G, N, K]")
    G, M, K = XQ.shape
    G2, N, K2 = WQ.shape
    if G2 != G or K2 != K:
        raise ValueError(f"shape mismatch: XQ {tuple(XQ.shape)} vs WQ {tuple(WQ.shape)}")
    if K % 128 or N % 128:
        raise ValueError(f"block scaling needs K and N to be multiples of 128 (N={N}, K={K})")
    _on_gpu(XQ, "XQ")
    _on_gpu(WQ, "WQ")
    _check(x_scale, "x_scale", torch.float32, (G, M, K // 128))
    _check(w_scale, "w_scale", torch.float32, (G, N // 128, K // 128))
    if out is None:
        out = torch.empty((G, M, N), dtype=torch.bfloat16, device=XQ.device)
    _check(out, "out", torch.bfloat16, (G, M, N))
    st = getattr(_lib.load(), fn_name)(XQ.data_ptr(), WQ.data_ptr(), x_scale.data_ptr(), w_scale.data_ptr(),
                                       out.data_ptr(), G, M, N, K, _stream(XQ.device))
    _lib.check(st, fn_name)
    return out


def _groupwise(fn_name, XQ, WQ, x_scale, w_scale, M_sizes, out, meta_name="M_sizes", meta_dtype=torch.int64):
    XQ = _bytes(XQ, "XQ")
    WQ = _bytes(WQ, "WQ")
    if XQ.dim() != 2 or WQ.dim() != 3:
        raise ValueError("XQ must be [total_M, K] and WQ [G, N, K]")
    total_M, K = XQ.shape
    G, N, K2 = WQ.shape
    if K2 != K:
        raise ValueError(f"K mismatch: XQ has {K}, WQ has {K2}")
    if K % 128 or N % 128:
        raise ValueError(f"block scaling needs K and N to be multiples of 128 (N={N}, K={K})")
    _on_gpu(XQ, "XQ")
    _on_gpu(WQ, "WQ")
    _check(x_scale, "x_scale", torch.float32, (total_M, K // 128))
    _check(w_scale, "w_scale", torch.float32, (G, N // 128, K // 128))
    _check(M_sizes, meta_name, meta_dtype, (G,))
    if out is None:
        out = torch.empty((total_M, N), dtype=torch.bfloat16, device=XQ.device)
    _check(out, "out", torch.bfloat16, (total_M, N))
    st = getattr(_lib.load(), fn_name)(XQ.data_ptr(), WQ.data_ptr(), x_scale.data_ptr(), w_scale.data_ptr(),
                                       M_sizes.data_ptr(), out.data_ptr(), G, total_M, N, K, _stream(XQ.device))
    _lib.check(st, fn_name)
    return out


def f8f8bf16_shuffle_b(WQ, out=None):
    """Rearranges WQ [G, N, K] into the pre-shuffled layout (same shape and bytes)."""
    WQ = _bytes(WQ, "WQ")
    if WQ.dim() != 3:
        raise ValueError("WQ must be [G, N, K]")
    G, N, K = WQ.shape
    _on_gpu(WQ, "WQ")
    if out is None:
        out = torch.empty_like(WQ)
    _check(out, "out", torch.uint8, (G, N, K))
    st = _lib.load().f8f8bf16_shuffle_b(WQ.data_ptr(), out.data_ptr(), G, N, K, _stream(WQ.device))
    _lib.check(st, "f8f8bf16_shuffle_b")
    return out


def f8f8bf16_quantize_rowwise(X, XQ=None, x_scale=None):
    """Rowwise fp8 quantisation of bf16 activations X [rows, K]: returns (XQ uint8
    [rows, K] e4m3fn codes, x_scale float32 [rows]) (see include/fp8gg.h)."""
    if X.dim() != 2:
        raise ValueError("X must be [rows, K]")
    rows, K = X.shape
    _check(X, "X", torch.bfloat16, (rows, K))
    if XQ is None:
        XQ = torch.empty((rows, K), dtype=torch.uint8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty((rows,), dtype=torch.float32, device=X.device)
    XQ = _bytes(XQ, "XQ")
    _check(XQ, "XQ", torch.uint8, (rows, K))
    _check(x_scale, "x_scale", torch.float32, (rows,))
    st = _lib.load().f8f8bf16_quantize_rowwise(X.data_ptr(), XQ.data_ptr(), x_scale.data_ptr(), rows, K,
                                              _stream(X.device))
    _lib.check(st, "f8f8bf16_quantize_rowwise")
    return XQ, x_scale
