"""GPU parity of qgemm_w4_nk (weights stored [N, K/8], scales [N, K/group_size])
against the oracle.

Modular page "multistage_gemm_q": the configuration's transpose_b flag; the
values are those of qgemm_w4 with transposed operands. Bars as test_gpu_w4.py:
|gpu - oracle| <= 1e-2 (|oracle| + 1) (the bf16 prefill path: the bound of its
weight rounding), unit rows bit-exact, and the prefill kernel bit-identical to
qgemm_w4 on the transposed operands (it only stages them differently).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, assert_close, bf16v, dev16, dev32, f16v, host16, say
from test_gpu_w4 import SENT, SENT_BF16, assert_within, bf16_weight_bound

pytestmark = pytest.mark.gpu


def nk_of(w):
    return np.ascontiguousarray(w.b.T), np.ascontiguousarray(w.scales.T)


def run(lib, w, nk=True, env=None, variant=None):
    M, N, K = w.shape
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    b, s = nk_of(w) if nk else (w.b, w.scales)
    out = Guarded((M, N), tdt, SENT_BF16 if w.dtype == "bf16" else SENT)
    if variant is not None:
        os.environ[env] = str(variant)
    try:
        fn = lib.qgemm_w4_nk if nk else lib.qgemm_w4
        fn(out.view, dev16(w.a, tdt), dev32(b), dev16(s, tdt), w.group_size)
    finally:
        if variant is not None:
            del os.environ[env]
    got = host16(out.view)
    assert out.bands_intact(), "write outside C"
    return got


def check(lib, w, what, rows=None, **kw):
    M, N, K = w.shape
    say(f"[w4-nk] {what}: M={M} N={N} K={K} gs={w.group_size} {w.dtype} {kw}")
    got = run(lib, w, **kw)
    b, s = nk_of(w)
    a = w.a if rows is None else w.a[rows]
    if rows is not None:
        got = got[rows]
    ref = oracle.qgemm_w4_nk(a, b, s, w.group_size, dtype=w.dtype)
    if w.dtype == "bf16" and M > 16:
        return assert_within(bf16v(got), bf16v(ref), bf16_weight_bound(w, rows), what)
    v = bf16v if w.dtype == "bf16" else f16v
    return assert_close(v(got), v(ref), what=what)


DECODE_SHAPES = [(16, 256, 512, 128), (3, 264, 384, 128), (13, 72, 256, 32), (7, 520, 512, 64), (1, 4104, 1024, 128),
                 (2, 192, 8192, 256), (9, 128, 1024, 32)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("variant", range(9, 16))
def test_decode_variants(gpu, lib, variant, dtype):
    for (M, N, K, gs) in DECODE_SHAPES:
        w = synth.w4_inputs(M, N, K, seed=M * 7 + N, group_size=gs, dtype=dtype)
        check(lib, w, f"decode v{variant}", env="QG_W4_DECODE_VARIANT", variant=variant)


PREFILL_SHAPES = [(48, 256, 512, 128), (17, 64, 256, 128), (100, 136, 96, 32), (257, 1000, 448, 64),
                  (300, 264, 1024, 256), (129, 8, 128, 128)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("variant", [11, 13, 14, 15, 16, 17])
def test_prefill_variants_and_identity_with_qgemm_w4(gpu, lib, variant, dtype):
    for (M, N, K, gs) in PREFILL_SHAPES:
        w = synth.w4_inputs(M, N, K, seed=M + N + K, group_size=gs, dtype=dtype)
        check(lib, w, f"prefill v{variant}", env="QG_W4_PREFILL_VARIANT", variant=variant)
        a = run(lib, w, nk=True, env="QG_W4_PREFILL_VARIANT", variant=variant)
        b = run(lib, w, nk=False, env="QG_W4_PREFILL_VARIANT", variant=variant)
        assert np.array_equal(a, b), f"v{variant} {M}x{N}x{K}: differs from qgemm_w4 on the transposed operands"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_full_size(gpu, lib, dtype):
    for c in synth.W4_DECODE:
        check(lib, synth.w4_inputs(**c, dtype=dtype), f"decode full M={c['M']}")
    w = synth.w4_inputs(**synth.W4_PREFILL, dtype=dtype)
    M = w.shape[0]
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(3).choice(M, 48, replace=False)]))
    say("  diagnostics", check(lib, w, "prefill full", rows=rows))


def test_unit_rows_bit_exact(gpu, lib):
    """A = I_K (decode: its first 16 rows): each output is the rounded weight (q - 8) * s."""
    K, N, gs = 512, 320, 128
    for dtype, one in (("f16", 0x3C00), ("bf16", 0x3F80)):
        for M in (16, K):
            w = synth.w4_inputs(M, N, K, seed=6, group_size=gs, dtype=dtype)
            w.a = np.zeros((M, K), np.uint16)
            w.a[np.arange(M), np.arange(M)] = one
            got = run(lib, w)
            b, s = nk_of(w)
            assert np.array_equal(got, oracle.qgemm_w4_nk(w.a, b, s, gs, dtype=dtype)), (dtype, M)


def test_rejects_two_stage_prefill(gpu, lib):
    w = synth.w4_inputs(64, 256, 512, seed=1)
    b, s = nk_of(w)
    out = torch.empty((64, 256), dtype=torch.float16, device="cuda")
    os.environ["QG_W4_PREFILL_VARIANT"] = "12"
    try:
        st = lib.qgemm_w4_nk(out, dev16(w.a, torch.float16), dev32(b), dev16(s, torch.float16), 128,
                             raise_on_error=False)
    finally:
        del os.environ["QG_W4_PREFILL_VARIANT"]
    assert st == lib.QG.ERR_UNSUPPORTED
