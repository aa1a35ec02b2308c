"""Seeded random-shape parity sweep of every entry point against the oracle.

The fixed-shape tests pick their sizes by hand; this one draws them (row counts
on and off the tile heights, any multiple of 16 columns, depths of one to many
quantisation groups, 1 to 19 experts with skipped rows, ragged sequences with
cached history, keys or keys and values, bf16 or e4m3 cache and hidden rows,
every epilogue flag, both types, both weight layouts) so that an
edge a hand-picked list misses still meets the common bar
|gpu - oracle| <= 1e-2 (|oracle| + 1). Each case prints its shape before it runs.

Both sides round their result to the output type once, so a case can differ by
one unit in the last place where the exact value sits near a rounding boundary:
for bf16 that is at most 2^(e-7) / (1e-2 (2^e + 1)) < 0.79 of the bar, which is
why the bar, not bit equality, is the criterion here.
"""
import numpy as np
import pytest

import synth
import test_gpu_grouped_epilogue as tg
import test_gpu_kv_cache as tkv
import test_gpu_w4_epilogue as te
import test_gpu_w4_nk as tn
from gpu_util import say

pytestmark = pytest.mark.gpu

DENSE_M = [1, 2, 3, 4, 5, 8, 9, 15, 16, 17, 31, 33, 64, 100, 127, 129, 200, 257, 300]


def dense_case(lib, rng, i, nk):
    dtype = str(rng.choice(["f16", "bf16"]))
    gs = int(rng.choice([32, 64, 128, 256]))
    M = int(rng.choice(DENSE_M))
    N = int(16 * rng.integers(1, 80))
    K = int(gs * rng.integers(1, max(2, 2048 // gs)))
    w = synth.w4_inputs(M, N, K, seed=1000 + i, group_size=gs, dtype=dtype)
    if nk:
        tn.check(lib, w, f"random {i}")
    else:
        te.check(lib, w, int(rng.integers(0, 8)), 5000 + i, f"random {i}")


def grouped_case(lib, rng, i, w4):
    E = int(rng.integers(1, 20))
    T = int(rng.integers(1, 700))
    N = int(16 * rng.integers(1, 40))
    flags = int(rng.integers(0, 8))
    skip = float(rng.uniform(0, 0.5))
    if w4:
        dtype = str(rng.choice(["f16", "bf16"]))
        gs = int(rng.choice([32, 64, 128, 256]))
        K = int(gs * rng.integers(1, max(2, 1024 // gs)))
        say(f"[random {i}] grouped w4 E={E} T={T} N={N} K={K} gs={gs} {dtype} flags={flags}")
        d = synth.grouped_w4_inputs(seed=2000 + i, E=E, T=T, K=K, N=N, skip_frac=skip, group_size=gs, dtype=dtype)
        tg.run_w4(lib, d, flags, 6000 + i)
    else:
        K = int(8 * rng.integers(1, 128))
        tb = bool(rng.integers(0, 2))
        say(f"[random {i}] grouped bf16 E={E} T={T} N={N} K={K} transpose_b={tb} flags={flags}")
        d = synth.grouped_inputs(seed=3000 + i, E=E, T=T, K=K, N=N, skip_frac=skip)
        tg.run_bf16(lib, d, flags, 7000 + i, transpose_b=tb)


def kproj_case(lib, rng, i):
    B = int(rng.integers(1, 9))
    lens = [int(x) for x in rng.integers(0, 300, B)]
    lens[int(rng.integers(0, B))] = int(rng.integers(1, 300))
    history = [int(x) for x in rng.integers(0, 200, B)]
    D = int(rng.choice([64, 128]))
    hkv = int(rng.choice([2, 4])) if D == 64 else int(rng.choice([1, 2, 4]))
    planes = int(rng.integers(1, 3))
    cache = str(rng.choice(["bf16", "fp8"]))
    qgran = int(rng.choice([g for g in (32, 64, 128) if g <= D]))
    hidden = str(rng.choice(["bf16", "fp8"]))
    k = tkv.kv_inputs(4000 + i, lens, cache_lengths=history, Kh=int(128 * rng.integers(1, 9)), hkv=hkv, D=D,
                      page_size=int(rng.choice([1, 16, 32, 64, 128])), planes=planes, cache=cache, qgran=qgran,
                      layer=int(rng.integers(0, 2)), hidden=hidden)
    tkv.check(lib, k, f"random {i}")


@pytest.mark.parametrize("seed", range(4))
def test_random_shapes(gpu, lib, seed):
    rng = np.random.default_rng(100 + seed)
    for j in range(36):
        i = 36 * seed + j
        kind = int(rng.integers(0, 6))
        if kind <= 1:
            dense_case(lib, rng, i, nk=False)
        elif kind == 2:
            dense_case(lib, rng, i, nk=True)
        elif kind <= 4:
            grouped_case(lib, rng, i, w4=(kind == 3))
        else:
            kproj_case(lib, rng, i)
