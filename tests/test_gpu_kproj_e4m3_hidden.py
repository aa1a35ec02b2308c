"""GPU parity of the K-projection calls with e4m3 hidden rows (the page's dtype
parameter for hidden_state), against the oracle.

Both operands are then e4m3 and one v_mfma_scale_f32_16x16x128_f8f6f4 sums a
128-term block. That instruction does not round its sum once from the exact
value: an in-bounds probe (random e4m3 operands, 51,200 outputs) found 60
results equal to the fp32 rounding of the exact sum and errors up to 7e-5 of
the block's magnitude sum. Bars: untouched cache bytes bit-exact; bf16 outputs
within 1e-2 (|oracle| + 1); e4m3 caches within half a code step of the exact
product widened by E = 2^-12 M (M: the sum of the terms' magnitudes), and scales
within E / 448 of the oracle's (test_gpu_kv_cache.check); bit-exact outputs
where every block sum is exact (one nonzero term).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bf16v, dev8, dev16, dev32, devf32, host16, say
from oracle import numerics as nm
from test_gpu_kv_cache import TILE_LENS, check, kv_inputs, run_gpu, run_ref

pytestmark = pytest.mark.gpu


def test_keys_bf16_cache_ragged(gpu, lib):
    check(lib, kv_inputs(1, (5, 17, 3), planes=1, hidden="fp8"), "tiny")
    check(lib, kv_inputs(2, (100, 1, 64, 65, 0, 130), cache_lengths=(0, 3, 17, 128, 5, 250), planes=1,
                         hidden="fp8"), "ragged+history")
    check(lib, kv_inputs(3, (300,), Kh=512, hkv=4, D=64, page_size=128, planes=1, hidden="fp8"), "one seq")
    check(lib, kv_inputs(4, (1, 2, 3, 70), Kh=128, hkv=1, D=128, page_size=1, layers=1, layer=0, planes=1,
                         hidden="fp8"), "page size 1")


@pytest.mark.parametrize("qgran", [32, 128])
def test_keys_and_values_both_caches(gpu, lib, qgran):
    check(lib, kv_inputs(10 + qgran, (100, 1, 64, 65, 0, 130), cache_lengths=(0, 3, 17, 128, 5, 250),
                         hidden="fp8"), "fused bf16 cache")
    check(lib, kv_inputs(11 + qgran, (100, 1, 64, 65, 0, 130), cache_lengths=(0, 3, 17, 128, 5, 250),
                         hidden="fp8", cache="fp8", qgran=qgran), "fused e4m3 cache")


def test_e4m3_weight_codes_bit_exact(gpu, lib):
    """Hidden rows are unit vectors (code 0x38 = 1.0): each token reads back one
    weight row, and every finite weight code appears: bit-exact bf16 outputs."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    k = kv_inputs(5, (254,), Kh=256, hkv=1, D=128, page_size=256, layers=1, layer=0, planes=1, hidden="fp8")
    w = np.zeros((256, 128), np.uint8)
    w[:254, 0] = codes
    w[:254, 1:] = codes[::-1, None]
    h = np.zeros((254, 256), np.uint8)
    h[np.arange(254), np.arange(254)] = 0x38
    got, _ = run_gpu(lib, k, hidden=h, weight=w, input_scale=np.ones((254, 2), np.float32),
                     weight_scale=np.ones((2, 1), np.float32))
    ref, _ = run_ref(k, hidden_bits=h, weight_codes=w, input_scale=np.ones((254, 2), np.float32),
                     weight_scale=np.ones((2, 1), np.float32))
    assert np.array_equal(got, ref)


def test_e4m3_hidden_codes_bit_exact(gpu, lib):
    """Every finite hidden code in column 0 of a token, times a unit weight."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    k = kv_inputs(6, (254,), Kh=256, hkv=1, D=128, page_size=256, layers=1, layer=0, planes=1, hidden="fp8")
    h = np.zeros((254, 256), np.uint8)
    h[:, 0] = codes
    h[:, 200] = codes[::-1]
    w = np.zeros((256, 128), np.uint8)
    w[0, :64] = 0x38
    w[200, 64:] = 0x38
    over = dict(input_scale=np.ones((254, 2), np.float32), weight_scale=np.ones((2, 1), np.float32))
    got, _ = run_gpu(lib, k, hidden=h, weight=w, **over)
    ref, _ = run_ref(k, hidden_bits=h, weight_codes=w, **over)
    assert np.array_equal(got, ref)


# every row-tile height (48, 96, 144 rows)
@pytest.mark.parametrize("i", range(3))
def test_tile_heights(gpu, lib, i):
    check(lib, kv_inputs(40 + i, TILE_LENS[1024][i], Kh=256, hkv=8, D=128, page_size=128, planes=1, hidden="fp8"),
          "keys bf16")
    check(lib, kv_inputs(50 + i, TILE_LENS[2048][i], Kh=384, hkv=8, D=128, page_size=16, cache="fp8", qgran=64,
                         hidden="fp8"), "fused e4m3, odd stages")


def test_full_size(gpu, lib):
    """The K-projection workload (T = 4312, hidden 4096 -> 1024) with e4m3 hidden rows
    (one scale per token per 128 columns), keys only and keys + values into an e4m3 cache."""
    say("  diagnostics", check(lib, synth.kproj_inputs(hidden="fp8"), "full keys"))
    say("  diagnostics", check(lib, synth.kproj_inputs(hidden="fp8", planes=2, cache="fp8", qgran=128),
                               "full fused e4m3 cache"))


def test_long_hidden(gpu, lib):
    """More than 32 scale blocks of K (input scales refilled every 32 blocks)."""
    check(lib, kv_inputs(90, (100, 1, 64), Kh=33 * 128, planes=1, hidden="fp8"), "Kh=4224 keys bf16")
    check(lib, kv_inputs(91, (150, 20), Kh=65 * 128, cache="fp8", qgran=64, hidden="fp8"), "Kh=8320 kv e4m3")


def test_determinism(gpu, lib):
    k = kv_inputs(80, (200, 31), cache="fp8", qgran=32, hidden="fp8")
    a, sa = run_gpu(lib, k)
    b, sb = run_gpu(lib, k)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)
