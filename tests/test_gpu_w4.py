"""GPU parity of qgemm_w4 (through the C ABI) against the CPU oracle.

Modular page "multistage_gemm_q": group_size K elements per scale,
pack_factor 4-bit codes per uint32. Float outputs: |gpu - oracle| <=
1e-2 (|oracle| + 1) per element; unpacked weights: bit-exact."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, assert_close, bf16v, dev16, dev32, f16v, host16, say

pytestmark = pytest.mark.gpu

SENT = 0x7E00  # fp16 NaN pattern: never produced by the kernels
SENT_BF16 = 0xFFC1  # bf16 NaN pattern: never produced by the kernels


def run_w4(lib, w: synth.W4Inputs, variant_env=None, variant=None):
    M, N, K = w.shape
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    a = dev16(w.a, tdt)
    b = dev32(w.b)
    s = dev16(w.scales, tdt)
    out = Guarded((M, N), tdt, SENT_BF16 if w.dtype == "bf16" else SENT)
    if variant is not None:
        os.environ[variant_env] = str(variant)
    try:
        lib.qgemm_w4(out.view, a, b, s, w.group_size)
    finally:
        if variant is not None:
            del os.environ[variant_env]
    got = host16(out.view)
    assert out.bands_intact(), "write outside C"
    return got


def bf16_weight_bound(w, rows=None):
    """Per-element error bound of the bf16 prefill path, from its arithmetic: each
    weight (q - 8) * s is rounded to bf16 (unit roundoff u = 2^-8) before the
    fp32-accumulated MFMAs (slack K * 2^-24 <= 2^-12 relative to |A| . |W| for
    K <= 4096), and both the kernel's and the oracle's results are rounded to
    bf16: |gpu - oracle| <= u * (|A| . |W|) + 2u * |exact| + 2^-12 * (|A| . |W|)."""
    a = np.abs(oracle.numerics.decode_bf16(w.a if rows is None else w.a[rows]))
    wt = np.abs(oracle.w4.dequant_w4(w.b, w.scales, w.group_size, dtype="bf16"))
    mag = a @ wt
    exact = np.abs(oracle.w4.qgemm_w4_f64(w.a if rows is None else w.a[rows], w.b, w.scales, w.group_size,
                                          dtype="bf16"))
    u = 2.0 ** -8
    return u * mag + 2 * u * exact + 2.0 ** -12 * mag + 1e-30


def assert_within(got, ref, bound, what):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond the bf16-weight bound, worst "
                           f"{float((err / bound).max()):.3f} x bound")
    return {"max_err_over_bound": float((err / bound).max())}


def check(lib, w, what, **kw):
    M, N, K = w.shape
    say(f"[w4] {what}: M={M} N={N} K={K} gs={w.group_size} {w.dtype} {kw}")
    got = run_w4(lib, w, **kw)
    ref = oracle.qgemm_w4(w.a, w.b, w.scales, w.group_size, dtype=w.dtype)
    if w.dtype == "bf16" and M > 16:
        # the prefill path rounds the weights to bf16: the bound derived from that
        return assert_within(bf16v(got), bf16v(ref), bf16_weight_bound(w), what)
    v = bf16v if w.dtype == "bf16" else f16v
    return assert_close(v(got), v(ref), what=what)


DECODE_VARIANTS = range(16)


def test_tiny_config(gpu, lib):
    w = synth.w4_inputs(**synth.W4_TINY)
    check(lib, w, "tiny")


@pytest.mark.parametrize("variant", DECODE_VARIANTS)
def test_decode_variants_tiny_and_ragged(gpu, lib, variant):
    for (M, N, K, gs) in [(16, 256, 512, 128), (3, 264, 384, 128), (13, 72, 256, 32), (7, 520, 512, 64),
                          (16, 8, 256, 256), (1, 4104, 1024, 128), (5, 1024, 2048, 64), (2, 192, 8192, 256),
                          (9, 128, 1024, 32)]:
        w = synth.w4_inputs(M, N, K, seed=M * 7 + N, group_size=gs)
        check(lib, w, f"decode v{variant}", variant_env="QG_W4_DECODE_VARIANT", variant=variant)


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

PREFILL_VARIANTS = range(20)


@pytest.mark.parametrize("variant", PREFILL_VARIANTS)
def test_prefill_variants_ragged(gpu, lib, variant):
    for (M, N, K, gs) in [(48, 256, 512, 128), (17, 64, 256, 128), (100, 136, 96, 32), (257, 1000, 448, 64),
                          (300, 264, 1024, 256), (129, 8, 128, 128)]:
        w = synth.w4_inputs(M, N, K, seed=M + N + K, group_size=gs)
        check(lib, w, f"prefill v{variant}", variant_env="QG_W4_PREFILL_VARIANT", variant=variant)


@pytest.mark.parametrize("cfg", [synth.W4_PREFILL, synth.W4_SQUARE_PREFILL], ids=["N11008", "N4096"])
def test_prefill_full_size_sampled_rows(gpu, lib, cfg):
    """Full-size launch; the oracle recomputes 48 sampled rows (each row of C depends
    only on its row of A) plus first and last rows."""
    w = synth.w4_inputs(**cfg)
    M, N, K = w.shape
    say(f"[w4] prefill full M={M} N={N} K={K}")
    got = run_w4(lib, w)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(0).choice(M, 48, replace=False)]))
    ref = oracle.qgemm_w4(w.a[rows], w.b, w.scales, w.group_size)
    d = assert_close(f16v(got[rows]), f16v(ref), what="prefill-full")
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

BF16_DECODE_VARIANTS = range(9, 16)     # the LDS-staged decode kernel
BF16_PREFILL_VARIANTS = range(11, 20)   # the fourth prefill design


@pytest.mark.parametrize("variant", BF16_DECODE_VARIANTS)
def test_bf16_decode_variants(gpu, lib, variant):
    for (M, N, K, gs) in [(16, 256, 512, 128), (3, 264, 384, 128), (13, 72, 256, 32), (1, 4104, 1024, 128),
                          (2, 192, 8192, 256), (9, 128, 1024, 64)]:
        w = synth.w4_inputs(M, N, K, seed=M * 5 + N, group_size=gs, dtype="bf16")
        check(lib, w, f"bf16 decode v{variant}", variant_env="QG_W4_DECODE_VARIANT", variant=variant)


@pytest.mark.parametrize("variant", BF16_PREFILL_VARIANTS)
def test_bf16_prefill_variants(gpu, lib, variant):
    for (M, N, K, gs) in [(48, 256, 512, 128), (17, 64, 256, 128), (100, 136, 96, 32), (257, 1000, 448, 64),
                          (129, 8, 128, 128)]:
        w = synth.w4_inputs(M, N, K, seed=M + N + K + 1, group_size=gs, dtype="bf16")
        check(lib, w, f"bf16 prefill v{variant}", variant_env="QG_W4_PREFILL_VARIANT", variant=variant)


def test_bf16_full_size(gpu, lib):
    """Decode M = 1, 4, 16 at N = K = 4096 and the 2048 x 11008 x 4096 prefill
    (48 sampled rows) with bf16 activations, scales and output."""
    for c in synth.W4_DECODE:
        check(lib, synth.w4_inputs(**c, dtype="bf16"), f"bf16 decode M={c['M']}")
    w = synth.w4_inputs(**synth.W4_PREFILL, dtype="bf16")
    M = w.shape[0]
    got = run_w4(lib, w)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(1).choice(M, 48, replace=False)]))
    ref = oracle.qgemm_w4(w.a[rows], w.b, w.scales, w.group_size, dtype="bf16")
    say("  diagnostics", assert_within(bf16v(got[rows]), bf16v(ref), bf16_weight_bound(w, rows), "bf16 prefill-full"))


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
