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
"""
from __future__ import annotations

import numpy as np

from .numerics import decode_f16, round_to_f16, f16_bits_of


def _check_rank2(*arrs):
    for a in arrs:
        if np.ndim(a) != 2:
            raise ValueError("multistage_gemm_q: input tensors must be rank-2")


def dequant_w4(b_packed, scales_bits, group_size: int, pack_factor: int = 8) -> np.ndarray:
    """Packed codes + fp16 scales -> float64 weights W [K, N] (exact)."""
    _check_rank2(b_packed, scales_bits)
    if pack_factor != 8:
        raise ValueError("only 8 four-bit codes per uint32 exist")
    b = np.asarray(b_packed, dtype=np.uint32)
    kp, n = b.shape
    K = kp * pack_factor
    if K % group_size:
        raise ValueError("K must be a multiple of group_size")
    s = decode_f16(scales_bits)
    if s.shape != (K // group_size, n):
        raise ValueError("scales must be [K/group_size, N]")
    shifts = (4 * np.arange(pack_factor, dtype=np.uint32))[None, :, None]
    q = ((b[:, None, :] >> shifts) & np.uint32(0xF)).astype(np.int64)   # [K/8, 8, N]
    q = q.reshape(K, n)
    group_of_k = np.arange(K) // group_size
    return (q - 8).astype(np.float64) * s[group_of_k, :]


def qgemm_w4_f64(a_bits, b_packed, scales_bits, group_size: int, pack_factor: int = 8) -> np.ndarray:
    """Unrounded fp64 product A . W."""
    _check_rank2(a_bits, b_packed, scales_bits)
    a = decode_f16(a_bits)
    w = dequant_w4(b_packed, scales_bits, group_size, pack_factor)
    if a.shape[1] != w.shape[0]:
        raise ValueError("A is [M, K] and B unpacks to [K, N]")
    return a @ w


def qgemm_w4(a_bits, b_packed, scales_bits, group_size: int, pack_factor: int = 8) -> np.ndarray:
    """C = round_fp16(A . dequant(B)) as fp16 bit patterns [M, N]."""
    c = round_to_f16(qgemm_w4_f64(a_bits, b_packed, scales_bits, group_size, pack_factor))
    assert np.all(np.isfinite(c)), "fp16 overflow in the reference result"
    return f16_bits_of(c)
