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
  * weight is OCP fp8 E4M3; hidden is bf16 (the workload's type) or E4M3 (the
    page's separate dtype parameter; a uint8 array here), and is multiplied by
    its scale in full precision.
  * Cache layout blocks[L][2][P][S][Hkv][D] with plane 0 = keys, 1 = values;
    page_table[b][j] is the physical page of the j-th logical page of sequence b;
    token j of sequence b goes to position cache_lengths[b] + j (appended after
    the cached history); cache_lengths itself is not updated.
  * The result is rounded to bf16 (round-to-nearest-even); every byte of the
    cache that no token targets keeps its prior value.
  * Quantized cache (kv_collection's scale_dtype_ / quantization_granularity_
    parameters, otherwise undescribed): e4m3 codes with one float32 scale per
    run of G head-dim elements of a cache row. The writer takes the fp32 value x
    of each element, amax = max |x| over the run, s = amax / 448 and code =
    e4m3(x / s) (nearest even; 0 when amax = 0), each division in float32, the
    precision in which the GPU kernel decides the codes.
  * Values (kv_matmul_ragged_paged_scale): the same product with the value
    weights appended to the key weights ([W_k | W_v]); columns N..2N-1 go to
    plane 1 of the same (page, slot).
"""
from __future__ import annotations

import numpy as np

from .numerics import decode_bf16, decode_e4m3, encode_e4m3, round_to_bf16, bf16_bits_of


def kproj_exact(hidden_bits, weight_codes, input_scale, weight_scale,
                granularity=(1, 128, 128)) -> np.ndarray:
    """(hidden * input_scale) . (weight * weight_scale) in float64, [T, N]; hidden is
    bf16 bits (uint16) or E4M3 codes (uint8)."""
    gm, gn, gk = granularity
    if (gm, gn, gk) != (1, 128, 128):
        raise ValueError("only (1, 128, 128) scale granularity is defined here")
    hb = np.asarray(hidden_bits)
    h = decode_e4m3(hb) if hb.dtype == np.uint8 else decode_bf16(hb)
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
    return x @ wf


def kproj_rows(hidden_bits, weight_codes, input_scale, weight_scale,
               granularity=(1, 128, 128)) -> np.ndarray:
    """round_bf16( (hidden * input_scale) . (weight * weight_scale) ) as bf16 bits [T, N]."""
    r = round_to_bf16(kproj_exact(hidden_bits, weight_codes, input_scale, weight_scale, granularity))
    assert np.all(np.isfinite(r)), "bf16 overflow in the reference result"
    return bf16_bits_of(r)


def quantize_runs(values, G: int):
    """Rows of values -> (e4m3 codes, float32 scales [.., n / G]): per run of G
    elements s = amax / 448 and code = e4m3(x / s), in float32 (code 0 and
    s = 0 for an all-zero run)."""
    x32 = np.asarray(values, dtype=np.float64).astype(np.float32)
    T, n = x32.shape
    runs = x32.reshape(T, n // G, G)
    amax = np.abs(runs).max(axis=2)
    s = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0))
    v = np.where(s[:, :, None] > 0, runs / safe[:, :, None], np.float32(0.0)).astype(np.float32)
    return encode_e4m3(v.astype(np.float64)).reshape(T, n), s


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


def _project_into_cache(hidden_bits, row_offsets, weight_codes, input_scale, weight_scale, blocks_in,
                        cache_lengths, page_table, layer_idx, granularity, planes, scales_in, qgran):
    blocks = np.array(blocks_in, copy=True)
    if blocks.ndim != 6:
        raise ValueError("cache blocks are [L, 2, P, S, Hkv, D]")
    L, two, P, S, Hkv, D = blocks.shape
    if not (0 <= layer_idx < L):
        raise ValueError("layer_idx out of range")
    exact = kproj_exact(hidden_bits, weight_codes, input_scale, weight_scale, granularity)
    n = Hkv * D
    if exact.shape[1] != planes * n:
        raise ValueError("weight columns must equal planes * num_kv_heads * head_size")
    offs = np.asarray(row_offsets, dtype=np.int64)
    if offs[-1] != exact.shape[0]:
        raise ValueError("input_row_offsets must end at sum(seq_lens)")
    _, page, slot = token_slots(row_offsets, cache_lengths, page_table, S)
    fp8 = blocks.dtype == np.uint8
    scales = np.array(scales_in, copy=True) if fp8 else None
    for plane in range(planes):
        part = exact[:, plane * n:(plane + 1) * n]
        if fp8:
            if D % qgran:
                raise ValueError("quantization granularity must divide head_size")
            codes, sc = quantize_runs(part, qgran)
        else:
            r = round_to_bf16(part)
            assert np.all(np.isfinite(r)), "bf16 overflow in the reference result"
            codes = bf16_bits_of(r)
        for t in range(exact.shape[0]):
            blocks[layer_idx, plane, page[t], slot[t]] = codes[t].reshape(Hkv, D)
            if fp8:
                scales[layer_idx, plane, page[t], slot[t]] = sc[t].reshape(Hkv, D // qgran)
    return (blocks, scales) if fp8 else blocks


def k_matmul_ragged_paged_scale(hidden_bits, row_offsets, weight_codes, input_scale,
                                weight_scale, blocks_bits, cache_lengths, page_table,
                                layer_idx: int, granularity=(1, 128, 128), scales=None,
                                quantization_granularity: int = 0):
    """Returns the updated cache: bf16 bits shaped like blocks_bits, or, for an e4m3
    cache (uint8 blocks), the pair (codes, float32 scales)."""
    return _project_into_cache(hidden_bits, row_offsets, weight_codes, input_scale, weight_scale, blocks_bits,
                               cache_lengths, page_table, layer_idx, granularity, 1, scales,
                               quantization_granularity)


def kv_matmul_ragged_paged_scale(hidden_bits, row_offsets, weight_codes, input_scale,
                                 weight_scale, blocks_bits, cache_lengths, page_table,
                                 layer_idx: int, granularity=(1, 128, 128), scales=None,
                                 quantization_granularity: int = 0):
    """Keys and values at once: weight_codes is [Kh, 2N] = [W_k | W_v]; columns
    N..2N-1 are written to plane 1. Returns as k_matmul_ragged_paged_scale."""
    return _project_into_cache(hidden_bits, row_offsets, weight_codes, input_scale, weight_scale, blocks_bits,
                               cache_lengths, page_table, layer_idx, granularity, 2, scales,
                               quantization_granularity)
