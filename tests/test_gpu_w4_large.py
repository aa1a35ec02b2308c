"""GPU parity of qgemm_w4 at a weight size beyond 32-bit byte offsets.

K = 16384 and N = 557056 make the packed B 4.56 GB (the second half of its
packed rows lies past byte 2^32): the decode kernel indexes with 64-bit
offsets, and the tiled prefill kernel rebuilds its B and scale descriptors at
each stage's first packed row, so its 32-bit buffer offsets stay within one
stage. The oracle recomputes sampled columns (each column of C depends only on
that column of B and of the scales), spread over the whole width and
concentrated at the end, where the offsets are largest. fp16 and bf16, plain
and with the fixed epilogue. Floats: |gpu - oracle| <= 1e-2 (|oracle| + 1).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, bf16v, dev16, f16v, host16, say

pytestmark = pytest.mark.gpu

K, N, GS = 16384, 557056, 128


@pytest.fixture(scope="module")
def big_weights(gpu):
    rng = np.random.default_rng(77)
    say(f"[w4-large] drawing B [{K // 8}, {N}] ({K // 8 * N * 4 / 1e9:.2f} GB)")
    b = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
    s32 = rng.uniform(0.005, 0.02, size=(K // GS, N)).astype(np.float32)
    s = {"f16": s32.astype(np.float16).view(np.uint16),
         "bf16": torch.from_numpy(s32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)}
    bd = torch.from_numpy(b.view(np.int32)).cuda()
    sd = {k: dev16(v, torch.bfloat16 if k == "bf16" else torch.float16) for k, v in s.items()}
    cols = np.unique(np.concatenate([rng.choice(N, 40, replace=False), np.arange(N - 24, N), [0, 1, N // 2]]))
    yield b, s, bd, sd, cols
    del bd, sd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M", [3, 40])
def test_beyond_32bit_offsets(gpu, lib, big_weights, M, dtype):
    b, s, bd, sd, cols = big_weights
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    rng = np.random.default_rng(M)
    a32 = rng.standard_normal((M, K)).astype(np.float32)
    a = (a32.astype(np.float16).view(np.uint16) if dtype == "f16"
         else torch.from_numpy(a32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    c = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
    say(f"[w4-large] M={M} K={K} N={N} {dtype}")
    lib.qgemm_w4(c, dev16(a, tdt), bd, sd[dtype], GS)
    got = host16(c)
    ref = oracle.qgemm_w4(a, np.ascontiguousarray(b[:, cols]), np.ascontiguousarray(s[dtype][:, cols]), GS,
                          dtype=dtype)
    v = bf16v if dtype == "bf16" else f16v
    say("  diagnostics", assert_close(v(got[:, cols]), v(ref), what=f"M={M} {dtype} sampled columns"))
    assert np.all(np.isfinite(v(got))), "unwritten or non-finite outputs"


@pytest.mark.parametrize("M", [3, 40])
def test_beyond_32bit_offsets_epilogue(gpu, lib, big_weights, M):
    """Bias and residual (fp16) through the same launches."""
    b, s, bd, sd, cols = big_weights
    rng = np.random.default_rng(100 + M)
    a = rng.standard_normal((M, K)).astype(np.float16).view(np.uint16)
    bias = rng.standard_normal(N).astype(np.float16).view(np.uint16)
    res = rng.standard_normal((M, N)).astype(np.float16).view(np.uint16)
    c = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    say(f"[w4-large] epilogue M={M}")
    flags = lib.EPI_BIAS | lib.EPI_RESIDUAL
    lib.qgemm_w4_epilogue(c, dev16(a, torch.float16), bd, sd["f16"], flags, bias=dev16(bias, torch.float16),
                          residual=dev16(res, torch.float16), group_size=GS)
    got = host16(c)
    ref = oracle.qgemm_w4_epilogue(a, np.ascontiguousarray(b[:, cols]), np.ascontiguousarray(s["f16"][:, cols]), GS,
                                   flags, bias[cols], np.ascontiguousarray(res[:, cols]))
    say("  diagnostics", assert_close(f16v(got[:, cols]), f16v(ref), what=f"M={M} epilogue sampled columns"))
