"""Ragged, scaled K-projection into a paged KV cache: oracle.

Follows the Modular page "k_matmul_ragged_paged_scale" (nn / kv_cache_ragged):
  * Description: a matmul whose result is written into a mutable paged KV
    cache collection.
  * Args: hidden_state is (sum(seq_lens), num_heads*head_size);
    input_row_offsets is (batch_size+1,) and marks where each sequence starts;
    weight is (num_heads*head_size, num_kv_heads*head_size); input_scale is
    multiplied into the input and weight_scale into the weight; the layer's
    cache is picked by layer_idx.
  * Parameters: scales_granularity_mnk gives the scale block shape in (M, N, K).

Readings where the page is silent:
  * Granularity (1, 128, 128): input_scale is [T, K/128] (one per row per 128
    K-elements), weight_scale is [K/128, N/128] (one per 128x128 weight block,
    oriented like weight [K, N]).
  * weight is OCP fp8 E4M3; hidden is bf16 and is multiplied by its scale in
    full precision (the activations are not quantized).
  * Cache layout blocks[L][2][P][S][Hkv][D] with plane 0 = keys, 1 = values;
    page_table[b][j] is the physical page of the j-th logical page of sequence b;
    token j of sequence b goes to position cache_lengths[b] + j (appended after
    the cached history); cache_lengths itself is not updated.
  * The result is rounded to bf16 (round-to-nearest-even); every byte of the
    cache that no token targets keeps its prior value.
"""
from __future__ import annotations

import numpy as np

from .numerics import decode_bf16, decode_e4m3, round_to_bf16, bf16_bits_of


def kproj_rows(hidden_bits, weight_codes, input_scale, weight_scale,
               granularity=(1, 128, 128)) -> np.ndarray:
    """round_bf16( (hidden * input_scale) . (weight * weight_scale) ) as bf16 bits [T, N]."""
    gm, gn, gk = granularity
    if (gm, gn, gk) != (1, 128, 128):
        raise ValueError("only (1, 128, 128) scale granularity is defined here")
    h = decode_bf16(hidden_bits)
    w = decode_e4m3(weight_codes)
    T, K = h.shape
    K2, N = w.shape
    if K != K2 or K % gk or N % gn:
        raise ValueError("shape mismatch")
    isc = np.asarray(input_scale, dtype=np.float64)
    wsc = np.asarray(weight_scale, dtype=np.float64)
    if isc.shape != (T, K // gk) or wsc.shape != (K // gk, N // gn):
        raise ValueError("scale shape mismatch")
    x = h * isc[:, np.arange(K) // gk]
    wf = w * wsc[np.arange(K) // gk][:, np.arange(N) // gn]
    r = round_to_bf16(x @ wf)
    assert np.all(np.isfinite(r)), "bf16 overflow in the reference result"
    return bf16_bits_of(r)


def token_slots(row_offsets, cache_lengths, page_table, page_size: int):
    """For every token t: (sequence b, physical page, slot within the page)."""
    offs = np.asarray(row_offsets, dtype=np.int64)
    cl = np.asarray(cache_lengths, dtype=np.int64)
    pt = np.asarray(page_table, dtype=np.int64)
    T = int(offs[-1])
    seq = np.empty(T, dtype=np.int64)
    page = np.empty(T, dtype=np.int64)
    slot = np.empty(T, dtype=np.int64)
    for b in range(len(offs) - 1):
        t0, t1 = offs[b], offs[b + 1]
        j = np.arange(t1 - t0)
        pos = cl[b] + j
        seq[t0:t1] = b
        page[t0:t1] = pt[b, pos // page_size]
        slot[t0:t1] = pos % page_size
    return seq, page, slot


def k_matmul_ragged_paged_scale(hidden_bits, row_offsets, weight_codes, input_scale,
                                weight_scale, blocks_bits, cache_lengths, page_table,
                                layer_idx: int, granularity=(1, 128, 128)) -> np.ndarray:
    """Returns the updated cache (bf16 bits, same shape as blocks_bits)."""
    blocks = np.array(blocks_bits, dtype=np.uint16, copy=True)
    if blocks.ndim != 6:
        raise ValueError("cache blocks are [L, 2, P, S, Hkv, D]")
    L, two, P, S, Hkv, D = blocks.shape
    if not (0 <= layer_idx < L):
        raise ValueError("layer_idx out of range")
    kb = kproj_rows(hidden_bits, weight_codes, input_scale, weight_scale, granularity)
    if kb.shape[1] != Hkv * D:
        raise ValueError("weight columns must equal num_kv_heads * head_size")
    offs = np.asarray(row_offsets, dtype=np.int64)
    if offs[-1] != kb.shape[0]:
        raise ValueError("input_row_offsets must end at sum(seq_lens)")
    _, page, slot = token_slots(row_offsets, cache_lengths, page_table, S)
    for t in range(kb.shape[0]):
        blocks[layer_idx, 0, page[t], slot[t]] = kb[t].reshape(Hkv, D)
    return blocks
