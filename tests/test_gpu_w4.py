"""GPU parity of qgemm_w4 (through the C ABI) against the CPU oracle.

Modular page "multistage_gemm_q": group_size K elements per scale,
pack_factor 4-bit codes per uint32. Float outputs (fp16 and bf16): |gpu -
oracle| <= 1e-2 (|oracle| + 1) per element, every element of every output
compared; unpacked weights: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, assert_close, bf16v, dev16, dev32, f16v, host16, say

pytestmark = pytest.mark.gpu

SENT = 0x7E00  # fp16 NaN pattern: never produced by the kernels
SENT_BF16 = 0xFFC1  # bf16 NaN pattern: never produced by the kernels


def run_w4(lib, w: synth.W4Inputs):
    M, N, K = w.shape
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    a = dev16(w.a, tdt)
    b = dev32(w.b)
    s = dev16(w.scales, tdt)
    out = Guarded((M, N), tdt, SENT_BF16 if w.dtype == "bf16" else SENT)
    lib.qgemm_w4(out.view, a, b, s, w.group_size)
    got = host16(out.view)
    assert out.bands_intact(), "write outside C"
    return got


def check(lib, w, what):
    M, N, K = w.shape
    say(f"[w4] {what}: M={M} N={N} K={K} gs={w.group_size} {w.dtype}")
    got = run_w4(lib, w)
    ref = oracle.qgemm_w4(w.a, w.b, w.scales, w.group_size, dtype=w.dtype)
    v = bf16v if w.dtype == "bf16" else f16v
    return assert_close(v(got), v(ref), what=what)


# (M, N, K, group_size): tails in every dimension, K % 64 == 32, every group
# size, several tiles
DECODE_SHAPES = [(16, 256, 512, 128), (3, 264, 384, 128), (13, 72, 256, 32), (7, 520, 512, 64),
                 (16, 8, 256, 256), (1, 4104, 1024, 128), (5, 1024, 2048, 64), (2, 192, 8192, 256),
                 (9, 128, 1024, 32)]
# prefill: up to (129, 256, 64, 32) one workgroup of two K groups per CU (at most
# one tile per CU; with K = 64 the second group has no stage), the last three
# more tiles than CUs (two workgroups per CU); K % 64 == 32 takes the register-
# staged tile, whole 64-deep stages the direct-to-LDS one (fp16, [K/8, N])
PREFILL_SHAPES = [(48, 256, 512, 128), (17, 64, 256, 128), (100, 136, 96, 32), (257, 1000, 448, 64),
                  (300, 264, 1024, 256), (129, 8, 128, 128), (129, 256, 64, 32), (2100, 4104, 480, 32),
                  (2200, 4352, 512, 128), (2056, 4104, 320, 32)]


def test_tiny_config(gpu, lib):
    w = synth.w4_inputs(**synth.W4_TINY)
    check(lib, w, "tiny")


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decode_tiny_and_ragged(gpu, lib, shape):
    M, N, K, gs = shape
    w = synth.w4_inputs(M, N, K, seed=M * 7 + N, group_size=gs)
    check(lib, w, "decode")


@pytest.mark.parametrize("cfg", synth.W4_DECODE, ids=lambda c: f"M{c['M']}")
def test_decode_full_size(gpu, lib, cfg):
    w = synth.w4_inputs(**cfg)
    d = check(lib, w, "decode-full")
    say("  diagnostics", d)


def test_decode_unpacked_weights_bit_exact(gpu, lib):
    """Unit rows of A pick single K rows: C = round_fp16((q - 8) * s), compared bitwise."""
    N, K, gs = 4096, 4096, 128
    w = synth.w4_inputs(16, N, K, seed=2, a_seed=1)
    ks = np.array([0, 1, 7, 8, 127, 128, 129, 1000, 2047, 2048, 3071, 3072, 4000, 4093, 4094, 4095])
    a = np.zeros((16, K), np.uint16)
    a[np.arange(16), ks] = 0x3C00
    w.a = a
    got = run_w4(lib, w)
    ref = oracle.qgemm_w4(w.a, w.b, w.scales, gs)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 9, 15, 16])
def test_decode_every_row_count_class(gpu, lib, M):
    """Default decode path at each padded row count (1, 2, 4, 8, 16) and between."""
    w = synth.w4_inputs(M, 2048, 2048, seed=100 + M, group_size=128)
    check(lib, w, "decode rows")


def test_decode_zero_point_and_determinism(gpu, lib):
    w = synth.w4_inputs(16, 512, 1024, seed=9)
    w.b[:] = 0x88888888
    got = run_w4(lib, w)
    assert np.all(f16v(got) == 0.0)
    w2 = synth.w4_inputs(16, 4096, 4096, seed=2, a_seed=216)
    g1 = run_w4(lib, w2)
    g2 = run_w4(lib, w2)
    assert np.array_equal(g1, g2)


# ---------------------------------------------------------------- prefill (M > 16)

@pytest.mark.parametrize("shape", PREFILL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prefill_ragged(gpu, lib, shape):
    M, N, K, gs = shape
    w = synth.w4_inputs(M, N, K, seed=M + N + K, group_size=gs)
    check(lib, w, "prefill")


@pytest.mark.parametrize("cfg", [synth.W4_PREFILL, synth.W4_SQUARE_PREFILL], ids=["N11008", "N4096"])
def test_prefill_full_size(gpu, lib, cfg):
    """Full-size launch, every output element against the oracle."""
    w = synth.w4_inputs(**cfg)
    d = check(lib, w, "prefill-full")
    say("  diagnostics", d)


def test_prefill_unpacked_weights_bit_exact(gpu, lib):
    """A = I_K: every output is exactly round_fp16((q - 8) * s)."""
    K, N, gs = 512, 320, 128
    w = synth.w4_inputs(K, N, K, seed=4, group_size=gs)
    w.a = np.zeros((K, K), np.uint16)
    np.fill_diagonal(w.a, 0x3C00)
    got = run_w4(lib, w)
    ref = oracle.qgemm_w4(w.a, w.b, w.scales, gs)
    assert np.array_equal(got, ref)


def test_prefill_zero_point_and_determinism(gpu, lib):
    w = synth.w4_inputs(64, 256, 512, seed=10)
    w.b[:] = 0x88888888
    assert np.all(f16v(run_w4(lib, w)) == 0.0)
    w2 = synth.w4_inputs(300, 1024, 1024, seed=11)
    assert np.array_equal(run_w4(lib, w2), run_w4(lib, w2))


# ---------------------------------------------------------------- bf16 activations (a_type = c_type = bf16)

@pytest.mark.parametrize("shape", [s for s in DECODE_SHAPES if s[1] * s[2] <= 2 ** 22],
                         ids=lambda s: "x".join(map(str, s)))
def test_bf16_decode(gpu, lib, shape):
    M, N, K, gs = shape
    w = synth.w4_inputs(M, N, K, seed=M * 5 + N, group_size=gs, dtype="bf16")
    check(lib, w, "bf16 decode")


@pytest.mark.parametrize("shape", PREFILL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bf16_prefill(gpu, lib, shape):
    M, N, K, gs = shape
    w = synth.w4_inputs(M, N, K, seed=M + N + K + 1, group_size=gs, dtype="bf16")
    check(lib, w, "bf16 prefill")


@pytest.mark.parametrize("cfg", synth.W4_DECODE + [synth.W4_PREFILL, synth.W4_SQUARE_PREFILL],
                         ids=["M1", "M4", "M16", "prefill_N11008", "prefill_N4096"])
def test_bf16_full_size(gpu, lib, cfg):
    """bf16 activations, scales and output at the decode and both prefill sizes,
    every output element under the common bar."""
    d = check(lib, synth.w4_inputs(**cfg, dtype="bf16"), "bf16 full")
    say("  diagnostics", d)


def test_bf16_unit_rows_bit_exact(gpu, lib):
    """A = I_K (decode: the first 16 rows of it): each output is round_bf16((q - 8) * s)."""
    K, N, gs = 512, 320, 128
    for M in (16, K):
        w = synth.w4_inputs(M, N, K, seed=6, group_size=gs, dtype="bf16")
        w.a = np.zeros((M, K), np.uint16)
        w.a[np.arange(M), np.arange(M)] = 0x3F80   # bf16 1.0
        got = run_w4(lib, w)
        ref = oracle.qgemm_w4(w.a, w.b, w.scales, gs, dtype="bf16")
        assert np.array_equal(got, ref), f"M={M}"


def test_bf16_rejects_mixed_types(gpu, lib):
    w = synth.w4_inputs(16, 256, 512, seed=3, dtype="bf16")
    out = torch.empty((16, 256), dtype=torch.bfloat16, device="cuda")
    st = lib.qgemm_w4(out, dev16(w.a, torch.bfloat16), dev32(w.b), dev16(w.scales, torch.float16), 128,
                      raise_on_error=False)
    assert st == lib.QG.ERR_DTYPE
