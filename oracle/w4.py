"""W4A16 group-quantized GEMM oracle.

Follows the Modular page "multistage_gemm_q" (quantization / qmatmul_gpu):
C = A . B where B is a packed 4-bit weight buffer. Parameters section:
  * pack_factor: how many 4-bit elements one uint32 holds (8 here);
  * group_size:  how many K elements share one scale.
Raises section: inputs that are not rank-2 are an error.

Readings where the page is silent (each also a parity assumption):
  * B is [K / pack_factor, N] uint32, N contiguous; word (kp, n) holds the codes
    of rows k = pack_factor*kp + i, i = 0..7, code i in bits 4i..4i+3.
  * Scales are a separate fp16 [K / group_size, N] array; groups are contiguous
    runs of K starting at k = 0, so row k uses scale row k // group_size.
  * A code q in 0..15 stands for the weight (q - 8) * scale (no zero-point array).
  * The result is rounded to fp16 with round-to-nearest-even.
  * a_type / c_type (Parameters): activations, scales and result share one type,
    fp16 (the default) or bf16; the arithmetic is the same, only the decoding of
    the inputs and the rounding of the result change.
  * Epilogue (Parameters, the optional per-output-element function): a C ABI
    cannot carry a device function, so three fixed element-wise steps stand in
    for it, applied to the exact fp64 product before the single rounding:
    bias add over columns, then a SiLU-gated product of column pairs
    (2j, 2j+1) that halves N, then a residual add. SiLU is x / (1 + e^-x).
"""
from __future__ import annotations

import numpy as np

from .numerics import (bf16_bits_of, decode_bf16, decode_f16, f16_bits_of, round_to_bf16,
                       round_to_f16)

_DECODE = {"f16": decode_f16, "bf16": decode_bf16}
_ROUND = {"f16": (round_to_f16, f16_bits_of), "bf16": (round_to_bf16, bf16_bits_of)}


def _check_rank2(*arrs):
    for a in arrs:
        if np.ndim(a) != 2:
            raise ValueError("multistage_gemm_q: input tensors must be rank-2")


def dequant_w4(b_packed, scales_bits, group_size: int, pack_factor: int = 8, dtype: str = "f16") -> np.ndarray:
    """Packed codes + fp16 (or bf16) scales -> float64 weights W [K, N] (exact)."""
    _check_rank2(b_packed, scales_bits)
    if pack_factor != 8:
        raise ValueError("only 8 four-bit codes per uint32 exist")
    b = np.asarray(b_packed, dtype=np.uint32)
    kp, n = b.shape
    K = kp * pack_factor
    if K % group_size:
        raise ValueError("K must be a multiple of group_size")
    s = _DECODE[dtype](scales_bits)
    if s.shape != (K // group_size, n):
        raise ValueError("scales must be [K/group_size, N]")
    shifts = (4 * np.arange(pack_factor, dtype=np.uint32))[None, :, None]
    q = ((b[:, None, :] >> shifts) & np.uint32(0xF)).astype(np.int64)   # [K/8, 8, N]
    q = q.reshape(K, n)
    group_of_k = np.arange(K) // group_size
    return (q - 8).astype(np.float64) * s[group_of_k, :]


def qgemm_w4_f64(a_bits, b_packed, scales_bits, group_size: int, pack_factor: int = 8,
                 dtype: str = "f16") -> np.ndarray:
    """Unrounded fp64 product A . W."""
    _check_rank2(a_bits, b_packed, scales_bits)
    a = _DECODE[dtype](a_bits)
    w = dequant_w4(b_packed, scales_bits, group_size, pack_factor, dtype)
    if a.shape[1] != w.shape[0]:
        raise ValueError("A is [M, K] and B unpacks to [K, N]")
    return a @ w


def qgemm_w4(a_bits, b_packed, scales_bits, group_size: int, pack_factor: int = 8,
             dtype: str = "f16") -> np.ndarray:
    """C = round(A . dequant(B)) as fp16 (or bf16) bit patterns [M, N]."""
    rnd, bits_of = _ROUND[dtype]
    c = rnd(qgemm_w4_f64(a_bits, b_packed, scales_bits, group_size, pack_factor, dtype))
    assert np.all(np.isfinite(c)), "overflow in the reference result"
    return bits_of(c)


# Fixed epilogue flags (the C ABI's qgemm_w4_epilogue); they stand in for the
# page's optional per-element epilogue function.
EPI_BIAS, EPI_RESIDUAL, EPI_SILU_GATE = 1, 2, 4


def silu(x):
    """x * sigmoid(x) with sigmoid(x) = 1 / (1 + e^-x)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def fixed_epilogue(y, epilogue: int, bias=None, residual=None) -> np.ndarray:
    """The fixed steps on exact products y [M, N] (float64): y += bias [N]
    (EPI_BIAS); z = silu(y[:, 0::2]) * y[:, 1::2] (EPI_SILU_GATE, else z = y);
    z += residual [M, N_out] (EPI_RESIDUAL)."""
    if epilogue & EPI_BIAS:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    z = silu(y[:, 0::2]) * y[:, 1::2] if epilogue & EPI_SILU_GATE else y
    if epilogue & EPI_RESIDUAL:
        z = z + np.asarray(residual, dtype=np.float64)
    return z


def qgemm_w4_epilogue(a_bits, b_packed, scales_bits, group_size: int, epilogue: int, bias_bits=None,
                      residual_bits=None, pack_factor: int = 8, dtype: str = "f16") -> np.ndarray:
    """Y = A . dequant(B) in fp64; Y += bias (EPI_BIAS); Z = silu(Y[:, 0::2]) * Y[:, 1::2]
    (EPI_SILU_GATE, else Z = Y); Z += residual (EPI_RESIDUAL); one rounding to `dtype`."""
    dec = _DECODE[dtype]
    rnd, bits_of = _ROUND[dtype]
    y = qgemm_w4_f64(a_bits, b_packed, scales_bits, group_size, pack_factor, dtype)
    z = fixed_epilogue(y, epilogue, dec(bias_bits) if epilogue & EPI_BIAS else None,
                       dec(residual_bits) if epilogue & EPI_RESIDUAL else None)
    c = rnd(z)
    assert np.all(np.isfinite(c)), "overflow in the reference result"
    return bits_of(c)


def qgemm_w4_nk(a_bits, b_packed_nk, scales_nk, group_size: int, pack_factor: int = 8,
                dtype: str = "f16") -> np.ndarray:
    """The same product with B stored [N, K / pack_factor] and the scales
    [N, K / group_size] (the page's transpose_b configuration): word (n, kp) holds
    the codes of K rows pack_factor * kp + i of column n."""
    b = np.ascontiguousarray(np.asarray(b_packed_nk, dtype=np.uint32).T)
    s = np.ascontiguousarray(np.asarray(scales_nk, dtype=np.uint16).T)
    return qgemm_w4(a_bits, b, s, group_size, pack_factor, dtype)
