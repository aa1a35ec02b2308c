"""Grouped (MoE) GEMM oracle.

Follows the Modular page "grouped_matmul_sm100_persistent" (linalg /
grouped_matmul_sm100), Args section:
  * a_offsets: per-expert prefix sum of A row offsets (uint32);
  * expert_ids: per-group expert id (int32); negative entries skip the tile;
  * expert_usage_stats: its second entry is the number of active experts;
  * b: the weights, one matrix per expert; Parameters: transpose_b says
    whether each expert's matrix is stored transposed ([N, K]).

Readings where the page is silent:
  * Group g covers A rows a_offsets[g] .. a_offsets[g+1]-1 and uses expert
    expert_ids[g]; only groups g < expert_usage_stats[1] are processed.
  * Rows of a skipped group (negative id), and rows no processed group covers,
    are not written: C keeps whatever it held.
  * Empty groups and repeated expert ids are allowed; a_offsets[0] may be > 0.
  * The result is rounded to bf16 with round-to-nearest-even.
  * Epilogue (Parameters: the optional function on stored C fragments): the
    fixed steps of the W4 GEMM's epilogue, with one bias row per expert
    (bias [E, N]: the group's expert's row) and the residual shaped like C
    ([T, N_out], N_out = N / 2 with the SiLU gate).
"""
from __future__ import annotations

import numpy as np

from .numerics import decode_bf16, round_to_bf16, bf16_bits_of
from .w4 import fixed_epilogue, EPI_BIAS, EPI_RESIDUAL


def grouped_gemm(c_bits, a_bits, a_offsets, b_bits, expert_ids, usage_stats,
                 transpose_b: bool = True, epilogue: int = 0, bias_bits=None,
                 residual_bits=None) -> np.ndarray:
    """Returns the new C (bf16 bit patterns [T, N_out]); the input array is not modified."""
    out = np.array(c_bits, dtype=np.uint16, copy=True)
    a_off = np.asarray(a_offsets, dtype=np.int64)
    ids = np.asarray(expert_ids, dtype=np.int64)
    num_active = int(np.asarray(usage_stats)[1])
    if num_active > len(ids) or num_active + 1 > len(a_off):
        raise ValueError("active group count exceeds the routing tables")
    b = np.asarray(b_bits, dtype=np.uint16)
    for g in range(num_active):
        e = ids[g]
        if e < 0:
            continue
        r0, r1 = a_off[g], a_off[g + 1]
        if r1 <= r0:
            continue
        a = decode_bf16(a_bits[r0:r1])
        w = decode_bf16(b[e])
        prod = a @ (w.T if transpose_b else w)
        if epilogue:
            prod = fixed_epilogue(prod, epilogue,
                                  decode_bf16(np.asarray(bias_bits)[e]) if epilogue & EPI_BIAS else None,
                                  decode_bf16(np.asarray(residual_bits)[r0:r1]) if epilogue & EPI_RESIDUAL else None)
        r = round_to_bf16(prod)
        assert np.all(np.isfinite(r)), "bf16 overflow in the reference result"
        out[r0:r1] = bf16_bits_of(r)
    return out
