"""Grouped (MoE) GEMM oracle.

Follows the Modular page "grouped_matmul_sm100_persistent" (linalg /
grouped_matmul_sm100), Args section:
  * a_offsets: a prefix sum (uint32) of the row counts of A's groups;
  * expert_ids: the expert (int32) of each group; a group whose id is
    negative is not computed;
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
  * a_plane_splits (Parameters: split sizes per plane for the row offsets of
    A's planes in a fused LoRA QKV product; (0, 0) turns it off): two column
    counts (s0, s1). When not (0, 0), A holds three planes of T rows each
    ([3 T, K], T = rows of C; plane p is rows p T .. p T + T - 1, the LoRA
    shrink outputs of q, k and v), the N output columns split into
    [0, s0), [s0, s0 + s1) and [s0 + s1, N), and a column in range p reads
    its A rows from plane p: C[r, n] = sum_k A[p(n) T + r, k] W_e[n, k].
    Routing (a_offsets, expert_ids) indexes rows within a plane.
"""
from __future__ import annotations

import numpy as np

from .numerics import decode_bf16, round_to_bf16, bf16_bits_of
from .w4 import fixed_epilogue, EPI_BIAS, EPI_RESIDUAL


def plane_columns(a_plane_splits, n: int):
    """Column ranges [lo, hi) of A's planes, in plane order: one plane [0, n) for
    splits (0, 0), otherwise [0, s0), [s0, s0 + s1) and [s0 + s1, n)."""
    s0, s1 = (int(v) for v in a_plane_splits)
    if s0 == 0 and s1 == 0:
        return [(0, n)]
    if s0 < 0 or s1 < 0 or s0 + s1 > n:
        raise ValueError("a_plane_splits: the two split sizes must be >= 0 with s0 + s1 <= N")
    return [(0, s0), (s0, s0 + s1), (s0 + s1, n)]


def grouped_gemm(c_bits, a_bits, a_offsets, b_bits, expert_ids, usage_stats,
                 transpose_b: bool = True, epilogue: int = 0, bias_bits=None,
                 residual_bits=None, a_plane_splits=(0, 0)) -> np.ndarray:
    """Returns the new C (bf16 bit patterns [T, N_out]); the input array is not modified."""
    out = np.array(c_bits, dtype=np.uint16, copy=True)
    T = out.shape[0]
    b = np.asarray(b_bits, dtype=np.uint16)
    N = b.shape[1] if transpose_b else b.shape[2]
    planes = plane_columns(a_plane_splits, N)
    if np.shape(a_bits)[0] != len(planes) * T:
        raise ValueError("A must hold one block of T rows per plane")
    a_off = np.asarray(a_offsets, dtype=np.int64)
    ids = np.asarray(expert_ids, dtype=np.int64)
    num_active = int(np.asarray(usage_stats)[1])
    if num_active > len(ids) or num_active + 1 > len(a_off):
        raise ValueError("active group count exceeds the routing tables")
    for g in range(num_active):
        e = ids[g]
        if e < 0:
            continue
        r0, r1 = a_off[g], a_off[g + 1]
        if r1 <= r0:
            continue
        w = decode_bf16(b[e])
        wn = w if transpose_b else w.T          # [N, K]
        prod = np.zeros((r1 - r0, N))
        for p, (lo, hi) in enumerate(planes):
            a = decode_bf16(a_bits[p * T + r0:p * T + r1])
            prod[:, lo:hi] = a @ wn[lo:hi].T
        if epilogue:
            prod = fixed_epilogue(prod, epilogue,
                                  decode_bf16(np.asarray(bias_bits)[e]) if epilogue & EPI_BIAS else None,
                                  decode_bf16(np.asarray(residual_bits)[r0:r1]) if epilogue & EPI_RESIDUAL else None)
        r = round_to_bf16(prod)
        assert np.all(np.isfinite(r)), "bf16 overflow in the reference result"
        out[r0:r1] = bf16_bits_of(r)
    return out
