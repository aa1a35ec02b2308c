"""Grouped (MoE) W4A16 GEMM oracle (test infrastructure only).

Joins the two pages' definitions: the routing of "grouped_matmul_sm100_persistent"
(Args: a_offsets prefix sum of A rows per group, expert_ids with negative
entries skipping the group, expert_usage_stats[1] = number of groups to
process) applied to experts stored in the weight format of "multistage_gemm_q"
(Parameters: pack_factor 4-bit codes per uint32, group_size K elements per
scale). Neither page defines this combination; it is the plainest joint
reading:
  * expert e's weights are b_packed[e] ([K/8, N] uint32, code i of a word in
    bits 4i..4i+3 = K row 8*kp + i) with scales[e] ([K/group_size, N]); a code q
    stands for (q - 8) * scale;
  * group g < expert_usage_stats[1] with expert_ids[g] = e >= 0 sets
    C[a_offsets[g] .. a_offsets[g+1]-1] = round(A[those rows] . W_e), the
    product exact (fp64) and rounded once to the output type;
  * rows of skipped or unprocessed groups keep whatever C held.
  * the optional epilogue is the W4 GEMM's fixed steps with one bias row per
    expert (bias [E, N]) and the residual shaped like C ([T, N_out]).
  * A, the scales, C, bias and residual share one type: fp16 (the default) or
    bf16, as the W4 page's a_type / c_type parameters allow.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_bits_of, decode_bf16, decode_f16, f16_bits_of, round_to_bf16, round_to_f16
from .w4 import dequant_w4, fixed_epilogue, EPI_BIAS, EPI_RESIDUAL

_TYPES = {"f16": (decode_f16, round_to_f16, f16_bits_of), "bf16": (decode_bf16, round_to_bf16, bf16_bits_of)}


def grouped_gemm_w4(c_bits, a_bits, a_offsets, b_packed, scales_bits, expert_ids, usage_stats,
                    group_size: int, epilogue: int = 0, bias_bits=None, residual_bits=None,
                    dtype: str = "f16") -> np.ndarray:
    """Returns the new C (bit patterns of `dtype`, [T, N_out]); the input array is not modified."""
    dec, rnd, bits_of = _TYPES[dtype]
    out = np.array(c_bits, dtype=np.uint16, copy=True)
    a_off = np.asarray(a_offsets, dtype=np.int64)
    ids = np.asarray(expert_ids, dtype=np.int64)
    num_active = int(np.asarray(usage_stats)[1])
    if num_active > len(ids) or num_active + 1 > len(a_off):
        raise ValueError("active group count exceeds the routing tables")
    b = np.asarray(b_packed, dtype=np.uint32)
    s = np.asarray(scales_bits, dtype=np.uint16)
    if b.ndim != 3 or s.ndim != 3:
        raise ValueError("experts are [E, K/8, N] words and [E, K/group_size, N] scales")
    weights = {}
    for g in range(num_active):
        e = int(ids[g])
        if e < 0:
            continue
        r0, r1 = a_off[g], a_off[g + 1]
        if r1 <= r0:
            continue
        if e not in weights:
            weights[e] = dequant_w4(b[e], s[e], group_size, dtype=dtype)
        prod = dec(a_bits[r0:r1]) @ weights[e]
        if epilogue:
            prod = fixed_epilogue(prod, epilogue,
                                  dec(np.asarray(bias_bits)[e]) if epilogue & EPI_BIAS else None,
                                  dec(np.asarray(residual_bits)[r0:r1]) if epilogue & EPI_RESIDUAL else None)
        r = rnd(prod)
        assert np.all(np.isfinite(r)), "overflow in the reference result"
        out[r0:r1] = bits_of(r)
    return out
