"""CPU oracle for the three dequant-in-kernel GEMMs (test infrastructure only).

Plain, slow, obviously correct numpy fp64 implementations of what the GPU
library computes. Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import this package; the GPU library never
does, and this package imports nothing from it.

Sources (Modular MAX API reference pages):
  * "multistage_gemm_q" (quantization / qmatmul_gpu): W4A16 GEMM with
    group_size K-elements per scale and pack_factor 4-bit codes per uint32.
  * "grouped_matmul_sm100_persistent" (linalg / grouped_matmul_sm100):
    grouped GEMM routed by a_offsets / expert_ids / expert_usage_stats.
  * Both together: the grouped W4A16 GEMM (experts in the first page's
    packed format, routed as on the second).
  * "k_matmul_ragged_paged_scale" (nn / kv_cache_ragged): scaled matmul over
    ragged rows whose result is written into a paged KV cache.

Readings where the pages are silent are listed in each function's docstring.
"""
from .numerics import (round_to_f16, round_to_bf16, round_to, decode_f16, decode_bf16,
                       decode_e4m3, encode_e4m3, f16_bits_of, bf16_bits_of, F16, BF16, E4M3)
from .w4 import dequant_w4, qgemm_w4, qgemm_w4_nk, qgemm_w4_epilogue, silu, EPI_BIAS, EPI_RESIDUAL, EPI_SILU_GATE
from .grouped import grouped_gemm
from .grouped_w4 import grouped_gemm_w4
from .kproj import (k_matmul_ragged_paged_scale, kv_matmul_ragged_paged_scale, kproj_exact, kproj_rows,
                    quantize_runs, token_slots)

__all__ = [
    "round_to_f16", "round_to_bf16", "round_to", "decode_f16", "decode_bf16", "decode_e4m3",
    "encode_e4m3", "f16_bits_of", "bf16_bits_of", "F16", "BF16", "E4M3",
    "dequant_w4", "qgemm_w4", "qgemm_w4_nk", "qgemm_w4_epilogue", "silu", "EPI_BIAS", "EPI_RESIDUAL", "EPI_SILU_GATE",
    "grouped_gemm", "grouped_gemm_w4", "k_matmul_ragged_paged_scale", "kv_matmul_ragged_paged_scale",
    "kproj_exact", "kproj_rows", "quantize_runs",
    "token_slots",
]
