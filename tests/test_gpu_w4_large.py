"""GPU parity of qgemm_w4 at a weight size beyond 32-bit byte offsets.

K = 16384 and N = 557056 make the packed B 4.56 GB (the second half of its
packed rows lies past byte 2^32): the decode kernel indexes with 64-bit offsets
and the prefill call switches to the third design, whose loads do not use
32-bit buffer offsets. The oracle recomputes sampled columns (each column of C
depends only on that column of B and of the scales), spread over the whole
width and concentrated at the end, where the offsets are largest.
Floats: |gpu - oracle| <= 1e-2 (|oracle| + 1).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, dev16, f16v, host16, say

pytestmark = pytest.mark.gpu

K, N, GS = 16384, 557056, 128


@pytest.fixture(scope="module")
def big_weights(gpu):
    rng = np.random.default_rng(77)
    say(f"[w4-large] drawing B [{K // 8}, {N}] ({K // 8 * N * 4 / 1e9:.2f} GB)")
    b = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
    s = rng.uniform(0.005, 0.02, size=(K // GS, N)).astype(np.float16).view(np.uint16)
    bd = torch.from_numpy(b.view(np.int32)).cuda()
    sd = torch.from_numpy(s.view(np.int16)).cuda().view(torch.float16)
    cols = np.unique(np.concatenate([rng.choice(N, 40, replace=False), np.arange(N - 24, N), [0, 1, N // 2]]))
    yield b, s, bd, sd, cols
    del bd, sd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [3, 40])
def test_beyond_32bit_offsets(gpu, lib, big_weights, M):
    b, s, bd, sd, cols = big_weights
    rng = np.random.default_rng(M)
    a = rng.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    c = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    say(f"[w4-large] M={M} K={K} N={N}")
    lib.qgemm_w4(c, dev16(a, torch.float16), bd, sd, GS)
    got = host16(c)
    ref = oracle.qgemm_w4(a, np.ascontiguousarray(b[:, cols]), np.ascontiguousarray(s[:, cols]), GS)
    say("  diagnostics", assert_close(f16v(got[:, cols]), f16v(ref), what=f"M={M} sampled columns"))
    assert np.all(np.isfinite(f16v(got))), "unwritten or non-finite outputs"
