"""Seeded synthetic inputs shared by the CPU oracle, the GPU tests and the benchmark.

This module only draws random numbers and stores them in the bit layouts the
three operations take as input. It holds none of the operations' arithmetic
(no unpacking, no dequantization, no products, no rounding of results): every
array it returns is raw storage (uint16 bit patterns for fp16/bf16, uint8 codes
for fp8 e4m3, uint32 words for packed 4-bit weights, uint32/int32 index
tables), which both sides then interpret on their own.

Workloads (sizes and value distributions of the three pages' problems):

* W4A16 GEMM (Modular "multistage_gemm_q", Parameters: group_size,
  pack_factor): A fp16 ~ N(0,1); B as uniformly random 32-bit words, i.e.
  eight independent uniform 4-bit codes per word along K; scales fp16
  ~ U(0.005, 0.02), one per group_size K-rows per column.
* Grouped GEMM (Modular "grouped_matmul_sm100_persistent", Args: a_offsets,
  expert_ids, expert_usage_stats): 64 experts, 4096 routed rows split by
  multinomial counts, K=2048, N=1408, 10% of expert ids set to -1,
  A/B bf16 ~ N(0, 0.02).
* Ragged paged K-projection (Modular "k_matmul_ragged_paged_scale", Args):
  8 sequences of lengths U[1,1024], hidden 4096 bf16 ~ N(0,1), weight e4m3
  [4096,1024] from N(0,0.02) with one fp32 scale per 128x128 block
  (scale = block amax / 448), input scales ~ U(0.5, 2.0) per 128 K-elements
  per row, page size 128, random page table, 2 layers.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

__all__ = [
    "W4Inputs", "GroupedInputs", "KProjInputs",
    "w4_inputs", "grouped_inputs", "kproj_inputs",
    "f16_bits", "bf16_bits", "e4m3_codes",
    "W4_TINY", "W4_DECODE", "W4_PREFILL", "W4_SQUARE_PREFILL",
]


# ---------------------------------------------------------------------------
# storage conversions (library casts; the value is then only a bit pattern)
# ---------------------------------------------------------------------------

def f16_bits(x: np.ndarray) -> np.ndarray:
    """float64 array -> IEEE binary16 bit patterns (numpy's cast)."""
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float16)).view(np.uint16)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 array -> bfloat16 bit patterns (torch's float32 -> bfloat16 cast)."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float64 array -> OCP fp8 e4m3 ("fn") codes, saturated to +-448 first."""
    t = torch.from_numpy(np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


# ---------------------------------------------------------------------------
# W4A16
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class W4Inputs:
    a: np.ndarray          # uint16 [M, K]   fp16 (or bf16) bits
    b: np.ndarray          # uint32 [K/8, N] packed 4-bit codes
    scales: np.ndarray     # uint16 [K/group_size, N] fp16 (or bf16) bits
    group_size: int
    dtype: str = "f16"     # storage type of a and scales (and of the result)

    @property
    def shape(self):
        return self.a.shape[0], self.b.shape[1], self.a.shape[1]


def _bits(x, dtype: str):
    return bf16_bits(x) if dtype == "bf16" else f16_bits(x)


def w4_weights(seed: int, N: int, K: int, group_size: int = 128, dtype: str = "f16"):
    """Packed weights and scales for an N x K problem (draw order: words, scales)."""
    rng = np.random.default_rng(seed)
    b = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
    s = _bits(rng.uniform(0.005, 0.02, size=(K // group_size, N)), dtype)
    return b, s


def w4_activations(seed: int, M: int, K: int, dtype: str = "f16"):
    rng = np.random.default_rng(seed)
    return _bits(rng.standard_normal((M, K)), dtype)


def w4_inputs(M: int, N: int, K: int, seed: int = 1, a_seed: int | None = None,
              group_size: int = 128, dtype: str = "f16") -> W4Inputs:
    """W4A16 problem: weights from `seed`, activations from `a_seed` (default: seed+100);
    dtype "f16" or "bf16" stores the activations and scales (the same draws)."""
    b, s = w4_weights(seed, N, K, group_size, dtype)
    a = w4_activations(seed + 100 if a_seed is None else a_seed, M, K, dtype)
    return W4Inputs(a=a, b=b, scales=s, group_size=group_size, dtype=dtype)


def w4_epilogue_operands(seed: int, M: int, N_out: int, N: int, dtype: str = "f16"):
    """Bias [N] and residual [M, N_out] for the fixed W4 epilogues (draw order:
    bias, residual), standard normal in `dtype`."""
    rng = np.random.default_rng(seed)
    bias = _bits(rng.standard_normal(N), dtype)
    residual = _bits(rng.standard_normal((M, N_out)), dtype)
    return bias, residual


def grouped_epilogue_operands(seed: int, E: int, T: int, N_out: int, N: int, dtype: str = "bf16",
                              std: float = 1.0):
    """Per-expert bias [E, N] and residual [T, N_out] for the grouped GEMMs' fixed
    epilogues (draw order: bias, residual), normal with standard deviation `std`."""
    rng = np.random.default_rng(seed)
    bias = _bits(rng.normal(0.0, std, size=(E, N)), dtype)
    residual = _bits(rng.normal(0.0, std, size=(T, N_out)), dtype)
    return bias, residual


# Named W4 workloads: (M, N, K, weight seed, activation seed)
W4_TINY = dict(M=16, N=256, K=512, seed=1, a_seed=101)
W4_DECODE = [dict(M=m, N=4096, K=4096, seed=2, a_seed=200 + m) for m in (1, 4, 16)]
W4_PREFILL = dict(M=2048, N=11008, K=4096, seed=3, a_seed=103)
W4_SQUARE_PREFILL = dict(M=2048, N=4096, K=4096, seed=3, a_seed=103)


# ---------------------------------------------------------------------------
# Grouped (MoE) GEMM
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class GroupedInputs:
    a: np.ndarray           # uint16 [T, K] bf16 bits
    a_offsets: np.ndarray   # uint32 [G+1]
    b: np.ndarray           # uint16 [E, N, K] (transpose_b) or [E, K, N] bf16 bits
    expert_ids: np.ndarray  # int32 [G]
    usage: np.ndarray       # uint32 [2]: [0] max rows in a group, [1] active group count
    transpose_b: bool = True


def grouped_inputs(seed: int = 4, E: int = 64, T: int = 4096, K: int = 2048, N: int = 1408,
                   skip_frac: float = 0.10, transpose_b: bool = True, a_planes: int = 1) -> GroupedInputs:
    """Grouped workload. Draw order: counts, skipped groups, A, B. a_planes = 3
    draws A as three planes of T rows ([3 T, K], fused LoRA QKV inputs)."""
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(T, [1.0 / E] * E)
    a_off = np.zeros(E + 1, dtype=np.uint32)
    a_off[1:] = np.cumsum(counts)
    n_skip = int(np.floor(skip_frac * E))
    skip = rng.choice(E, n_skip, replace=False)
    ids = np.arange(E, dtype=np.int32)
    ids[skip] = -1
    a = bf16_bits(rng.normal(0.0, 0.02, size=(a_planes * T, K)))
    bshape = (E, N, K) if transpose_b else (E, K, N)
    b = bf16_bits(rng.normal(0.0, 0.02, size=bshape))
    usage = np.array([counts.max(), E], dtype=np.uint32)
    return GroupedInputs(a=a, a_offsets=a_off, b=b, expert_ids=ids, usage=usage,
                         transpose_b=transpose_b)


# ---------------------------------------------------------------------------
# Grouped (MoE) W4A16 GEMM
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class GroupedW4Inputs:
    a: np.ndarray           # uint16 [T, K] fp16 (or bf16) bits
    a_offsets: np.ndarray   # uint32 [G+1]
    b: np.ndarray           # uint32 [E, K/8, N] packed 4-bit codes
    scales: np.ndarray      # uint16 [E, K/group_size, N] fp16 (or bf16) bits
    expert_ids: np.ndarray  # int32 [G]
    usage: np.ndarray       # uint32 [2]: [0] max rows in a group, [1] active group count
    group_size: int = 128
    dtype: str = "f16"


def grouped_w4_inputs(seed: int = 6, E: int = 64, T: int = 4096, K: int = 2048, N: int = 1408,
                      skip_frac: float = 0.10, group_size: int = 128, dtype: str = "f16") -> GroupedW4Inputs:
    """Grouped W4A16 workload: the grouped workload's routing (multinomial counts,
    floor(skip_frac * E) skipped groups) with W4A16 operands (A ~ N(0,1), uniform
    4-bit codes, scales U(0.005, 0.02); A and the scales stored as `dtype`, fp16 or
    bf16, from the same draws). Draw order: counts, skipped groups, A, packed
    words, scales."""
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(T, [1.0 / E] * E)
    a_off = np.zeros(E + 1, dtype=np.uint32)
    a_off[1:] = np.cumsum(counts)
    n_skip = int(np.floor(skip_frac * E))
    skip = rng.choice(E, n_skip, replace=False)
    ids = np.arange(E, dtype=np.int32)
    ids[skip] = -1
    a = _bits(rng.standard_normal((T, K)), dtype)
    b = rng.integers(0, 2**32, size=(E, K // 8, N), dtype=np.uint32)
    s = _bits(rng.uniform(0.005, 0.02, size=(E, K // group_size, N)), dtype)
    usage = np.array([counts.max(), E], dtype=np.uint32)
    return GroupedW4Inputs(a=a, a_offsets=a_off, b=b, scales=s, expert_ids=ids, usage=usage,
                           group_size=group_size, dtype=dtype)


# ---------------------------------------------------------------------------
# Ragged paged K-projection
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class KProjInputs:
    hidden: np.ndarray        # [T, Kh]: uint16 bf16 bits, or uint8 e4m3 codes
    row_offsets: np.ndarray   # uint32 [B+1]
    weight: np.ndarray        # uint8  [Kh, planes * N] e4m3 codes
    input_scale: np.ndarray   # float32 [T, Kh/128]
    weight_scale: np.ndarray  # float32 [Kh/128, planes * N/128]
    blocks: np.ndarray        # [L, 2, P, S, Hkv, D] prior cache content: uint16 bf16 bits, or uint8 e4m3 codes
    cache_lengths: np.ndarray  # uint32 [B]
    page_table: np.ndarray    # uint32 [B, max_pages]
    layer_idx: int
    granularity: tuple = (1, 128, 128)
    scales: np.ndarray | None = None   # e4m3 cache: float32 [L, 2, P, S, Hkv, D / qgran]
    qgran: int = 0                     # e4m3 cache: head-dim elements per scale


def kproj_inputs(seed: int = 5, batch: int = 8, max_len: int = 1024, Kh: int = 4096,
                 n_kv_heads: int = 8, head_dim: int = 128, page_size: int = 128,
                 num_pages: int | None = None, num_layers: int = 2, layer_idx: int = 1,
                 cache_lengths=None, fill: int = 0xFFFF, lens=None,
                 max_pages: int | None = None, planes: int = 1, cache: str = "bf16",
                 qgran: int = 128, hidden: str = "bf16") -> KProjInputs:
    """K-projection workload. Draw order: lengths, hidden, weight, input scales, page table.

    planes = 2 draws [W_k | W_v] (2N columns) for the fused key/value projection.
    cache = "fp8" gives an e4m3 cache (prior codes 0x7F, a NaN the writers never
    produce) with float32 scales (prior value -1) per `qgran` head-dim elements.
    hidden = "fp8" stores the same normal draws as e4m3 codes with one float32
    input scale per token per 128 columns (amax / 448 of the block), in place of
    the uniform input scales (which are still drawn, keeping the draw order).

    `cache_lengths` (tokens already cached per sequence) defaults to zeros; the page
    table has `max_pages` entries per sequence (default: enough for max_len new tokens on
    top of the longest cache), filled from one random permutation of the physical pages.
    """
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(1, max_len + 1, batch)
    lens = np.asarray(lens, dtype=np.int64)
    batch = len(lens)
    offs = np.zeros(batch + 1, dtype=np.uint32)
    offs[1:] = np.cumsum(lens)
    T = int(offs[-1])
    N = n_kv_heads * head_dim
    h_real = rng.standard_normal((T, Kh))
    hidden_bits = bf16_bits(h_real)
    NW = planes * N
    w_real = rng.normal(0.0, 0.02, size=(Kh, NW))
    blk = w_real.reshape(Kh // 128, 128, NW // 128, 128)
    amax = np.abs(blk).max(axis=(1, 3)).astype(np.float32)
    ws = (amax / np.float32(448.0)).astype(np.float32)
    w_codes = e4m3_codes((blk / ws[:, None, :, None].astype(np.float64)).reshape(Kh, NW))
    in_scale = rng.uniform(0.5, 2.0, size=(T, Kh // 128)).astype(np.float32)
    if hidden == "fp8":
        hb = h_real.reshape(T, Kh // 128, 128)
        in_scale = (np.abs(hb).max(axis=2) / 448.0).astype(np.float32)
        hidden_bits = e4m3_codes((hb / in_scale[:, :, None].astype(np.float64)).reshape(T, Kh))
    if cache_lengths is None:
        cache_lengths = np.zeros(batch, dtype=np.uint32)
    cache_lengths = np.asarray(cache_lengths, dtype=np.uint32)
    need = (cache_lengths.astype(np.int64) + lens + page_size - 1) // page_size
    if max_pages is None:
        max_pages = int((int(cache_lengths.max(initial=0)) + max_len + page_size - 1) // page_size)
    assert max_pages >= need.max()
    if num_pages is None:
        num_pages = batch * max_pages
    assert num_pages >= batch * max_pages
    perm = rng.permutation(num_pages).astype(np.uint32)
    page_table = perm[: batch * max_pages].reshape(batch, max_pages).copy()
    shape = (num_layers, 2, num_pages, page_size, n_kv_heads, head_dim)
    scales = None
    if cache == "fp8":
        blocks = np.full(shape, 0x7F, dtype=np.uint8)
        scales = np.full(shape[:5] + (head_dim // qgran,), -1.0, dtype=np.float32)
    else:
        blocks = np.full(shape, fill, dtype=np.uint16)
    return KProjInputs(hidden=hidden_bits, row_offsets=offs, weight=w_codes, input_scale=in_scale,
                       weight_scale=ws, blocks=blocks, cache_lengths=cache_lengths,
                       page_table=page_table, layer_idx=layer_idx, scales=scales,
                       qgran=qgran if cache == "fp8" else 0)
