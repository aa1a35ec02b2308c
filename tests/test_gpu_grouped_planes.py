"""GPU parity of the grouped GEMM's a_plane_splits (fused LoRA QKV planes of A)
through the C ABI, against the oracle.

Modular page "grouped_matmul_sm100_persistent", Parameters: a_plane_splits
(split sizes per plane for the row offsets of A's planes; (0, 0) turns it
off). This library's reading: with splits (s0, s1), A holds three planes of T
rows and output columns [0, s0), [s0, s0 + s1), [s0 + s1, N) read planes 0, 1
and 2. Floats: |gpu - oracle| <= 1e-2 (|oracle| + 1) on every element; rows of
skipped groups keep their bits; a scaled-identity case is exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, assert_close, bf16v, dev16, dev32, host16, say
from oracle import numerics as nm

pytestmark = pytest.mark.gpu

SENT = 0xFFC1   # bf16 NaN pattern: never produced by the kernels
BIAS, RES, GATE = oracle.EPI_BIAS, oracle.EPI_RESIDUAL, oracle.EPI_SILU_GATE


def planes_inputs(seed, E, T, K, N, skip_frac=0.2):
    """The grouped recipe with A drawn for three planes ([3 T, K])."""
    d = synth.grouped_inputs(seed=seed, E=E, T=T, K=K, N=N, skip_frac=skip_frac, a_planes=3)
    return d, d.a


def run(lib, d, a3, splits, transpose_b=True, flags=0, seed=0, a_off=None, ids=None, usage=None):
    a_off = d.a_offsets if a_off is None else a_off
    ids = d.expert_ids if ids is None else ids
    usage = d.usage if usage is None else usage
    T = a3.shape[0] // 3
    E, N, _ = d.b.shape
    n_out = N // 2 if flags & GATE else N
    b = d.b if transpose_b else np.ascontiguousarray(d.b.transpose(0, 2, 1))
    out = Guarded((T, n_out), torch.bfloat16, SENT)
    args = (dev16(a3, torch.bfloat16), dev32(a_off), dev16(b, torch.bfloat16), dev32(np.asarray(ids, np.int32)),
            [int(v) for v in usage])
    bias = res = None
    if flags:
        bias, res = synth.grouped_epilogue_operands(seed, E, T, n_out, N, "bf16", std=0.02)
        lib.grouped_gemm_epilogue(out.view, *args, flags, bias=dev16(bias, torch.bfloat16) if flags & BIAS else None,
                                  residual=dev16(res, torch.bfloat16) if flags & RES else None,
                                  transpose_b=transpose_b, a_plane_splits=splits)
    else:
        lib.grouped_gemm(out.view, *args, transpose_b=transpose_b, a_plane_splits=splits)
    got = host16(out.view)
    assert out.bands_intact(), "write outside C"
    ref = oracle.grouped_gemm(np.full((T, n_out), SENT, np.uint16), a3, a_off, b, ids, usage,
                              transpose_b=transpose_b, epilogue=flags, bias_bits=bias, residual_bits=res,
                              a_plane_splits=splits)
    return got, ref


def check(lib, d, a3, splits, what, **kw):
    say(f"[planes] {what}: T={a3.shape[0] // 3} K={d.a.shape[1]} N={d.b.shape[1]} E={d.b.shape[0]} "
        f"splits={splits} {kw}")
    got, ref = run(lib, d, a3, splits, **kw)
    written = ref[:, 0] != SENT
    assert np.array_equal(got[:, 0] != SENT, written), "row routing differs"
    assert np.all(got[~written] == SENT), "a skipped row was written"
    diag = assert_close(bf16v(got[written]), bf16v(ref[written]), what=what)
    # the outputs are small next to the tolerance's absolute floor: the relative
    # RMS error catches a wrong plane or a dropped K tile
    assert diag["rel_rms"] < 3e-3, diag
    return diag


# (E, T, K, N, splits): boundaries inside and at 128-column tiles, empty planes, K / N tails
CASES = [(4, 200, 64, 256, (64, 64)), (5, 77, 40, 200, (40, 96)), (6, 300, 136, 520, (0, 264)),
         (3, 150, 72, 136, (136, 0)), (8, 600, 256, 1032, (512, 128)), (4, 90, 16, 48, (8, 8))]


@pytest.mark.parametrize("transpose_b", [True, False], ids=["ENK", "EKN"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[3]}_s{c[4][0]}_{c[4][1]}")
def test_ragged(gpu, lib, case, transpose_b):
    E, T, K, N, splits = case
    d, a3 = planes_inputs(10 + N, E, T, K, N)
    check(lib, d, a3, splits, "ragged", transpose_b=transpose_b)


@pytest.mark.parametrize("flags", [BIAS | RES, BIAS | GATE | RES], ids=["bias_res", "bias_gate_res"])
def test_epilogue(gpu, lib, flags):
    d, a3 = planes_inputs(20, 6, 400, 128, 528)
    check(lib, d, a3, (136, 264), "epilogue", flags=flags, seed=21)
    check(lib, d, a3, (136, 264), "epilogue [E,K,N]", flags=flags, seed=22, transpose_b=False)


def test_lora_expand_shape(gpu, lib):
    """A LoRA expand step: 8 adapters routed over 4096 rows, rank 16, q / k / v
    outputs 4096 / 1024 / 1024 wide."""
    d, a3 = planes_inputs(30, 8, 4096, 16, 6144, skip_frac=0.125)
    diag = check(lib, d, a3, (4096, 1024), "lora expand")
    say("  diagnostics", diag)


def test_planes_route_exactly(gpu, lib):
    """B[e] = c_e I and plane p of A = (p + 1) X: column n of a routed row is
    c_e (p(n) + 1) X[r, n], exact in bf16."""
    E, T, K = 4, 120, 256
    d = synth.grouped_inputs(seed=40, E=E, T=T, K=K, N=K, skip_frac=0.25, a_planes=3)
    x = np.random.default_rng(40).integers(-8, 9, size=(T, K)).astype(np.float64)
    a3 = nm.bf16_bits_of(np.concatenate([x, 2 * x, 3 * x]))
    fac = np.ldexp(1.0, np.arange(E) - 2)
    d.b = nm.bf16_bits_of(fac[:, None, None] * np.eye(K)[None])
    for splits in [(64, 128), (8, 240), (200, 0)]:
        for tb in (True, False):
            got, ref = run(lib, d, a3, splits, transpose_b=tb)
            assert np.array_equal(got, ref), (splits, tb)


def test_planes_off_match_the_plain_call(gpu, lib):
    d = synth.grouped_inputs(seed=50, E=5, T=300, K=128, N=200, skip_frac=0.2)
    T, N = d.a.shape[0], d.b.shape[1]
    o1 = Guarded((T, N), torch.bfloat16, SENT)
    o2 = Guarded((T, N), torch.bfloat16, SENT)
    args = (dev16(d.a, torch.bfloat16), dev32(d.a_offsets), dev16(d.b, torch.bfloat16), dev32(d.expert_ids),
            [int(v) for v in d.usage])
    lib.grouped_gemm(o1.view, *args)
    lib.grouped_gemm(o2.view, *args, a_plane_splits=(0, 0))
    assert np.array_equal(host16(o1.view), host16(o2.view))
