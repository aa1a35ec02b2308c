"""GPU parity of qgemm_w4_nk (weights stored [N, K/8], scales [N, K/group_size])
against the oracle.

Modular page "multistage_gemm_q": the configuration's transpose_b flag; the
values are those of qgemm_w4 with transposed operands. Bars as test_gpu_w4.py:
|gpu - oracle| <= 1e-2 (|oracle| + 1) on every element, unit rows bit-exact,
and the prefill kernel bit-identical to qgemm_w4 on the transposed operands (it
only stages them differently).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, assert_close, bf16v, dev16, dev32, f16v, host16, say
from test_gpu_w4 import DECODE_SHAPES, PREFILL_SHAPES, SENT, SENT_BF16

pytestmark = pytest.mark.gpu


def nk_of(w):
    return np.ascontiguousarray(w.b.T), np.ascontiguousarray(w.scales.T)


def run(lib, w, nk=True):
    M, N, K = w.shape
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    b, s = nk_of(w) if nk else (w.b, w.scales)
    out = Guarded((M, N), tdt, SENT_BF16 if w.dtype == "bf16" else SENT)
    fn = lib.qgemm_w4_nk if nk else lib.qgemm_w4
    fn(out.view, dev16(w.a, tdt), dev32(b), dev16(s, tdt), w.group_size)
    got = host16(out.view)
    assert out.bands_intact(), "write outside C"
    return got


def check(lib, w, what):
    M, N, K = w.shape
    say(f"[w4-nk] {what}: M={M} N={N} K={K} gs={w.group_size} {w.dtype}")
    got = run(lib, w)
    b, s = nk_of(w)
    ref = oracle.qgemm_w4_nk(w.a, b, s, w.group_size, dtype=w.dtype)
    v = bf16v if w.dtype == "bf16" else f16v
    return assert_close(v(got), v(ref), what=what)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [s for s in DECODE_SHAPES if s[1] * s[2] <= 2 ** 22],
                         ids=lambda s: "x".join(map(str, s)))
def test_decode(gpu, lib, shape, dtype):
    M, N, K, gs = shape
    check(lib, synth.w4_inputs(M, N, K, seed=M * 7 + N, group_size=gs, dtype=dtype), "decode")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", PREFILL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prefill_and_identity_with_qgemm_w4(gpu, lib, shape, dtype):
    M, N, K, gs = shape
    w = synth.w4_inputs(M, N, K, seed=M + N + K, group_size=gs, dtype=dtype)
    check(lib, w, "prefill")
    a = run(lib, w, nk=True)
    b = run(lib, w, nk=False)
    assert np.array_equal(a, b), f"{M}x{N}x{K}: differs from qgemm_w4 on the transposed operands"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("cfg", synth.W4_DECODE + [synth.W4_PREFILL], ids=["M1", "M4", "M16", "prefill"])
def test_full_size(gpu, lib, dtype, cfg):
    say("  diagnostics", check(lib, synth.w4_inputs(**cfg, dtype=dtype), "full"))


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
