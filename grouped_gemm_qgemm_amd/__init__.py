"""Python binding of libqgemm.so (the gfx950 dequant-in-kernel GEMM library).

Argument marshalling only: tensors are described to the C ABI in
include/qgemm.h (qg_tensor: pointer, dtype, rank, shape) and every step of the
computation runs in the library's HIP kernels. Torch tensors supply device
memory and the stream; nothing here computes a result. If the library is not
built, load() raises: there is no fallback path.

Entry points (same names as the C ABI):
    qgemm_w4(c, a, b_packed, scales, group_size=128, pack_factor=8)
    qgemm_w4_nk(c, a, b_packed_nk, scales_nk, group_size=128, pack_factor=8)
    qgemm_w4_epilogue(c, a, b_packed, scales, epilogue, bias=None, residual=None,
                      group_size=128, pack_factor=8)
    grouped_gemm(c, a, a_offsets, b, expert_ids, expert_usage_stats, transpose_b=True,
                 a_plane_splits=(0, 0))
    grouped_gemm_w4(c, a, a_offsets, b_packed, scales, expert_ids, expert_usage_stats,
                    group_size=128, pack_factor=8)
    grouped_gemm_epilogue(c, a, a_offsets, b, expert_ids, expert_usage_stats, epilogue, bias=None,
                          residual=None, transpose_b=True, a_plane_splits=(0, 0))
    grouped_gemm_w4_epilogue(..., epilogue, bias=None, residual=None, ...)
    k_matmul_ragged_paged_scale(hidden, input_row_offsets, weight, input_scale,
                                weight_scale, kv_blocks, cache_lengths, page_table,
                                layer_idx, scales_granularity_mnk=(1, 128, 128),
                                kv_scales=None, quantization_granularity=0)
    kv_matmul_ragged_paged_scale(... the same, weight = [W_k | W_v] ...)
Each returns None on success and raises QgError carrying the status otherwise.
Measurement yardsticks (include/qgemm_probe.h): read_contiguous, read_strips, mfma_loop,
empty_launch.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["load", "QgError", "qgemm_w4", "qgemm_w4_nk", "qgemm_w4_epilogue", "grouped_gemm", "grouped_gemm_w4",
           "grouped_gemm_epilogue", "grouped_gemm_w4_epilogue",
           "k_matmul_ragged_paged_scale", "kv_matmul_ragged_paged_scale", "status_string", "LIB_PATH", "QG", "EPI_BIAS", "EPI_RESIDUAL",
           "EPI_SILU_GATE"]

# qgemm_w4_epilogue flags
EPI_BIAS, EPI_RESIDUAL, EPI_SILU_GATE = 1, 2, 4

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqgemm.so")


class QG:
    OK, ERR_NULL, ERR_RANK, ERR_DTYPE, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_INVALID_ARG, ERR_LAUNCH = range(9)
    F16, BF16, F32, FP8_E4M3, U32, I32 = range(6)


MAX_RANK = 6


class QgTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int), ("rank", ctypes.c_int32),
                ("shape", ctypes.c_int64 * MAX_RANK)]


class QgPagedKV(ctypes.Structure):
    _fields_ = [("blocks", QgTensor), ("cache_lengths", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("max_pages_per_seq", ctypes.c_int64),
                ("scales", QgTensor), ("quantization_granularity", ctypes.c_int64)]


class QgError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"qgemm status {status}: {msg}")
        self.status = status


_lib = None

_TORCH_TO_QG = {
    torch.float16: QG.F16, torch.bfloat16: QG.BF16, torch.float32: QG.F32,
    torch.float8_e4m3fn: QG.FP8_E4M3, torch.uint32: QG.U32, torch.int32: QG.I32,
}


def load(path: str | None = None):
    """Load the built library (raises if it is missing; build with __graft_entry__.build())."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run python -m grouped_gemm_qgemm_amd.build")
    lib = ctypes.CDLL(p)
    T = ctypes.POINTER(QgTensor)
    lib.qgemm_w4.argtypes = [T, T, T, T, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.qgemm_w4.restype = ctypes.c_int
    lib.qgemm_w4_nk.argtypes = [T, T, T, T, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.qgemm_w4_nk.restype = ctypes.c_int
    lib.qgemm_w4_epilogue.argtypes = [T, T, T, T, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, T, T,
                                      ctypes.c_void_p]
    lib.qgemm_w4_epilogue.restype = ctypes.c_int
    lib.grouped_gemm.argtypes = [T, T, T, T, T, ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32,
                                 ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p]
    lib.grouped_gemm.restype = ctypes.c_int
    lib.grouped_gemm_w4.argtypes = [T, T, T, T, T, T, ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_void_p]
    lib.grouped_gemm_w4.restype = ctypes.c_int
    lib.grouped_gemm_epilogue.argtypes = [T, T, T, T, T, ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32,
                                          ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, T, T, ctypes.c_void_p]
    lib.grouped_gemm_epilogue.restype = ctypes.c_int
    lib.grouped_gemm_w4_epilogue.argtypes = [T, T, T, T, T, T, ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, T, T, ctypes.c_void_p]
    lib.grouped_gemm_w4_epilogue.restype = ctypes.c_int
    lib.k_matmul_ragged_paged_scale.argtypes = [T, T, T, T, T, ctypes.POINTER(ctypes.c_int32),
                                                ctypes.POINTER(QgPagedKV), ctypes.c_uint32, ctypes.c_void_p]
    lib.k_matmul_ragged_paged_scale.restype = ctypes.c_int
    lib.kv_matmul_ragged_paged_scale.argtypes = lib.k_matmul_ragged_paged_scale.argtypes
    lib.kv_matmul_ragged_paged_scale.restype = ctypes.c_int
    lib.qg_status_string.argtypes = [ctypes.c_int]
    lib.qg_status_string.restype = ctypes.c_char_p
    lib.qg_version.argtypes = []
    lib.qg_version.restype = ctypes.c_int32
    # measurement yardsticks (include/qgemm_probe.h)
    lib.qg_read_contiguous.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.qg_read_contiguous.restype = ctypes.c_int
    lib.qg_read_strips.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.qg_read_strips.restype = ctypes.c_int
    lib.qg_mfma_loop.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p]
    lib.qg_mfma_loop.restype = ctypes.c_int
    lib.qg_empty_launch.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.qg_empty_launch.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(s: int) -> str:
    return load().qg_status_string(s).decode()


def describe(t, dtype: int | None = None) -> QgTensor:
    """qg_tensor for a contiguous torch tensor (or None -> a NULL-data rank-0 record)."""
    d = QgTensor()
    if t is None:
        d.data = None
        d.dtype = dtype if dtype is not None else 0
        d.rank = 0
        return d
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    if t.dim() > MAX_RANK:
        raise ValueError("rank above 6")
    d.data = t.data_ptr() if t.numel() > 0 else (t.data_ptr() or None)
    d.dtype = dtype if dtype is not None else _TORCH_TO_QG.get(t.dtype, -1)
    d.rank = t.dim()
    for i, s in enumerate(t.shape):
        d.shape[i] = s
    return d


def _u32(t):
    """Tables of uint32 may be held in int32 or uint32 tensors."""
    return QG.U32 if t is not None and t.dtype in (torch.int32, torch.uint32) else None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(st: int):
    if st != QG.OK:
        raise QgError(st, status_string(st))


def qgemm_w4(c, a, b_packed, scales, group_size: int = 128, pack_factor: int = 8, stream=None,
             raise_on_error: bool = True) -> int:
    """C[M,N] (f16) = A[M,K] (f16) . dequant(B[K/8,N] u32, scales[K/gs,N] f16)."""
    lib = load()
    st = lib.qgemm_w4(ctypes.byref(describe(c)), ctypes.byref(describe(a)),
                      ctypes.byref(describe(b_packed, _u32(b_packed))), ctypes.byref(describe(scales)),
                      group_size, pack_factor, _stream(stream))
    if raise_on_error:
        _check(st)
    return st


def qgemm_w4_nk(c, a, b_packed, scales, group_size: int = 128, pack_factor: int = 8, stream=None,
                raise_on_error: bool = True) -> int:
    """qgemm_w4 with B stored [N, K/8] and the scales [N, K/group_size]."""
    lib = load()
    st = lib.qgemm_w4_nk(ctypes.byref(describe(c)), ctypes.byref(describe(a)),
                         ctypes.byref(describe(b_packed, _u32(b_packed))), ctypes.byref(describe(scales)),
                         group_size, pack_factor, _stream(stream))
    if raise_on_error:
        _check(st)
    return st


def qgemm_w4_epilogue(c, a, b_packed, scales, epilogue: int, bias=None, residual=None, group_size: int = 128,
                      pack_factor: int = 8, stream=None, raise_on_error: bool = True) -> int:
    """qgemm_w4 followed by a fixed epilogue (EPI_BIAS | EPI_SILU_GATE | EPI_RESIDUAL)."""
    lib = load()
    st = lib.qgemm_w4_epilogue(ctypes.byref(describe(c)), ctypes.byref(describe(a)),
                               ctypes.byref(describe(b_packed, _u32(b_packed))), ctypes.byref(describe(scales)),
                               group_size, pack_factor, int(epilogue),
                               ctypes.byref(describe(bias)) if bias is not None else None,
                               ctypes.byref(describe(residual)) if residual is not None else None,
                               _stream(stream))
    if raise_on_error:
        _check(st)
    return st


def _splits(a_plane_splits):
    return (ctypes.c_int32 * 2)(*[int(v) for v in a_plane_splits])


def grouped_gemm(c, a, a_offsets, b, expert_ids, expert_usage_stats, transpose_b: bool = True,
                 a_plane_splits=(0, 0), stream=None, raise_on_error: bool = True) -> int:
    """Rows of each active, non-skipped group g: C = A . B[expert_ids[g]]^T (bf16); with
    a_plane_splits (s0, s1) != (0, 0), A is [3 T, K] and column ranges [0, s0),
    [s0, s0 + s1), [s0 + s1, N) read planes 0, 1, 2 of A."""
    lib = load()
    usage = (ctypes.c_uint32 * 2)(*[int(v) for v in expert_usage_stats])
    st = lib.grouped_gemm(ctypes.byref(describe(c)), ctypes.byref(describe(a)),
                          ctypes.byref(describe(a_offsets, _u32(a_offsets))), ctypes.byref(describe(b)),
                          ctypes.byref(describe(expert_ids)), usage, int(bool(transpose_b)),
                          _splits(a_plane_splits), _stream(stream))
    if raise_on_error:
        _check(st)
    return st


def grouped_gemm_w4(c, a, a_offsets, b_packed, scales, expert_ids, expert_usage_stats, group_size: int = 128,
                    pack_factor: int = 8, stream=None, raise_on_error: bool = True) -> int:
    """Rows of each active, non-skipped group g: C = A . dequant(B[expert_ids[g]], scales[expert_ids[g]]) (f16)."""
    lib = load()
    usage = (ctypes.c_uint32 * 2)(*[int(v) for v in expert_usage_stats])
    st = lib.grouped_gemm_w4(ctypes.byref(describe(c)), ctypes.byref(describe(a)),
                             ctypes.byref(describe(a_offsets, _u32(a_offsets))),
                             ctypes.byref(describe(b_packed, _u32(b_packed))), ctypes.byref(describe(scales)),
                             ctypes.byref(describe(expert_ids)), usage, group_size, pack_factor, _stream(stream))
    if raise_on_error:
        _check(st)
    return st


def _opt(t):
    return ctypes.byref(describe(t)) if t is not None else None


def grouped_gemm_epilogue(c, a, a_offsets, b, expert_ids, expert_usage_stats, epilogue: int, bias=None,
                          residual=None, transpose_b: bool = True, a_plane_splits=(0, 0), stream=None,
                          raise_on_error: bool = True) -> int:
    """grouped_gemm followed by the fixed epilogue (bias [E, N] by expert, SiLU gate, residual)."""
    lib = load()
    usage = (ctypes.c_uint32 * 2)(*[int(v) for v in expert_usage_stats])
    st = lib.grouped_gemm_epilogue(ctypes.byref(describe(c)), ctypes.byref(describe(a)),
                                   ctypes.byref(describe(a_offsets, _u32(a_offsets))), ctypes.byref(describe(b)),
                                   ctypes.byref(describe(expert_ids)), usage, int(bool(transpose_b)),
                                   _splits(a_plane_splits), int(epilogue), _opt(bias), _opt(residual),
                                   _stream(stream))
    if raise_on_error:
        _check(st)
    return st


def grouped_gemm_w4_epilogue(c, a, a_offsets, b_packed, scales, expert_ids, expert_usage_stats, epilogue: int,
                             bias=None, residual=None, group_size: int = 128, pack_factor: int = 8, stream=None,
                             raise_on_error: bool = True) -> int:
    """grouped_gemm_w4 followed by the fixed epilogue (bias [E, N] by expert, SiLU gate, residual)."""
    lib = load()
    usage = (ctypes.c_uint32 * 2)(*[int(v) for v in expert_usage_stats])
    st = lib.grouped_gemm_w4_epilogue(ctypes.byref(describe(c)), ctypes.byref(describe(a)),
                                      ctypes.byref(describe(a_offsets, _u32(a_offsets))),
                                      ctypes.byref(describe(b_packed, _u32(b_packed))), ctypes.byref(describe(scales)),
                                      ctypes.byref(describe(expert_ids)), usage, group_size, pack_factor,
                                      int(epilogue), _opt(bias), _opt(residual), _stream(stream))
    if raise_on_error:
        _check(st)
    return st


def _paged_kv(kv_blocks, cache_lengths, page_table, kv_scales, quantization_granularity) -> QgPagedKV:
    kv = QgPagedKV()
    kv.blocks = describe(kv_blocks, QG.FP8_E4M3 if kv_blocks is not None and kv_blocks.dtype == torch.uint8 else None)
    kv.cache_lengths = cache_lengths.data_ptr() if cache_lengths is not None else None
    kv.page_table = page_table.data_ptr() if page_table is not None else None
    kv.max_pages_per_seq = page_table.shape[1] if page_table is not None and page_table.dim() == 2 else 0
    kv.scales = describe(kv_scales)
    kv.quantization_granularity = int(quantization_granularity)
    return kv


def _kv_call(fn, hidden, input_row_offsets, weight, input_scale, weight_scale, kv_blocks, cache_lengths,
             page_table, layer_idx, scales_granularity_mnk, kv_scales, quantization_granularity, stream,
             raise_on_error):
    gran = (ctypes.c_int32 * 3)(*[int(v) for v in scales_granularity_mnk])
    kv = _paged_kv(kv_blocks, cache_lengths, page_table, kv_scales, quantization_granularity)
    st = fn(ctypes.byref(describe(hidden)), ctypes.byref(describe(input_row_offsets, _u32(input_row_offsets))),
            ctypes.byref(describe(weight)), ctypes.byref(describe(input_scale)),
            ctypes.byref(describe(weight_scale)), gran, ctypes.byref(kv), int(layer_idx), _stream(stream))
    if raise_on_error:
        _check(st)
    return st


def k_matmul_ragged_paged_scale(hidden, input_row_offsets, weight, input_scale, weight_scale,
                                kv_blocks, cache_lengths, page_table, layer_idx: int,
                                scales_granularity_mnk=(1, 128, 128), kv_scales=None,
                                quantization_granularity: int = 0, stream=None,
                                raise_on_error: bool = True) -> int:
    """K rows = (hidden * input_scale) . (weight * weight_scale), written into the key
    plane of layer `layer_idx` of the paged cache `kv_blocks` [L, 2, P, S, Hkv, D]
    (bf16, or e4m3 codes held in float8_e4m3fn / uint8 with f32 `kv_scales`)."""
    return _kv_call(load().k_matmul_ragged_paged_scale, hidden, input_row_offsets, weight, input_scale,
                    weight_scale, kv_blocks, cache_lengths, page_table, layer_idx, scales_granularity_mnk,
                    kv_scales, quantization_granularity, stream, raise_on_error)


def kv_matmul_ragged_paged_scale(hidden, input_row_offsets, weight, input_scale, weight_scale,
                                 kv_blocks, cache_lengths, page_table, layer_idx: int,
                                 scales_granularity_mnk=(1, 128, 128), kv_scales=None,
                                 quantization_granularity: int = 0, stream=None,
                                 raise_on_error: bool = True) -> int:
    """Keys and values at once: weight = [W_k | W_v] ([Kh, 2 Hkv D]); planes 0 and 1."""
    return _kv_call(load().kv_matmul_ragged_paged_scale, hidden, input_row_offsets, weight, input_scale,
                    weight_scale, kv_blocks, cache_lengths, page_table, layer_idx, scales_granularity_mnk,
                    kv_scales, quantization_granularity, stream, raise_on_error)


def read_contiguous(src: torch.Tensor, sink: torch.Tensor, workgroups: int = 512, stream=None,
                    raise_on_error: bool = True) -> int:
    """Stream the bytes of `src` once (a measurement yardstick; writes nothing)."""
    st = load().qg_read_contiguous(src.data_ptr(), src.numel() * src.element_size(), int(workgroups),
                                   sink.data_ptr(), _stream(stream))
    if raise_on_error:
        _check(st)
    return st


def read_strips(src: torch.Tensor, strip_bytes: int, sink: torch.Tensor, stream=None,
                raise_on_error: bool = True) -> int:
    """Read a 2-D `src` one column strip of `strip_bytes` per workgroup, every row in
    order (a measurement yardstick; writes nothing)."""
    row_bytes = src.shape[1] * src.element_size()
    st = load().qg_read_strips(src.data_ptr(), src.shape[0], row_bytes, int(strip_bytes), sink.data_ptr(),
                               _stream(stream))
    if raise_on_error:
        _check(st)
    return st


MFMA_LOOP_KINDS = {"f16": 0, "bf16": 1, "e4m3": 2}
MFMA_LOOP_FLOPS = {0: 32768, 1: 32768, 2: 65536}   # FLOPs per MFMA of each kind


def mfma_loop(kind: int, iters: int, workgroups: int, clocks: torch.Tensor, sink: torch.Tensor, stream=None,
              raise_on_error: bool = True) -> int:
    """MFMA issue loop (a measurement yardstick): `clocks` is an int64 tensor of
    2 * workgroups elements that receives each workgroup's shader-clock cycles and
    100 MHz reference ticks across its loop."""
    if clocks.dtype != torch.int64 or clocks.numel() < 2 * int(workgroups):
        raise ValueError("clocks: int64 tensor of at least 2 * workgroups elements")
    st = load().qg_mfma_loop(int(kind), int(iters), int(workgroups), clocks.data_ptr(), sink.data_ptr(),
                             _stream(stream))
    if raise_on_error:
        _check(st)
    return st


def empty_launch(workgroups: int, threads: int, stream=None, raise_on_error: bool = True) -> int:
    """Launch a kernel that does nothing (a measurement yardstick)."""
    st = load().qg_empty_launch(int(workgroups), int(threads), _stream(stream))
    if raise_on_error:
        _check(st)
    return st
