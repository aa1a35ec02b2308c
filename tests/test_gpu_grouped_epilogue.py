"""GPU parity of grouped_gemm_epilogue and grouped_gemm_w4_epilogue (through the
C ABI) against the oracle.

The grouped page offers an optional function on the stored C fragments
(Parameters: elementwise_lambda_fn); the library's fixed steps stand in for it:
the bias row of the group's expert (bias [E, N]), a SiLU-gated product of column
pairs (2j, 2j+1) that halves N, a residual add, all before the one rounding.

Bars: routing (which rows are written) and every untouched row bit-exact;
every written output within 1e-2 (|oracle| + 1), gated ones included (every
kernel that computes a gated output keeps the weights exact in its MFMAs); and,
for the bf16 GEMM whose values are small next to the bar's floor, a relative RMS
error below 3e-3 over the rows.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import REL, Guarded, dev16, dev32, host16, say
from oracle import numerics as nm

pytestmark = pytest.mark.gpu

BIAS, RES, GATE = oracle.EPI_BIAS, oracle.EPI_RESIDUAL, oracle.EPI_SILU_GATE
SENT = {"bf16": 0xFFC1, "f16": 0x7E00}


def compare(got, ref, sent, dec, what, rel_rms=None):
    written = ref[:, 0] != sent
    assert np.array_equal(got[:, 0] != sent, written), f"{what}: row routing differs"
    assert np.all(got[~written] == sent), f"{what}: rows outside the groups changed"
    if not written.any():
        return {}
    g, r = dec(got[written]), dec(ref[written])
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    tol = REL * (np.abs(r) + 1.0)
    err = np.abs(g - r)
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond the tolerance, first "
                           f"{np.argwhere(bad)[:3].tolist()}, worst {float((err / tol).max()):.3f} x bound")
    rms = float(np.sqrt(np.mean(err ** 2)) / max(np.sqrt(np.mean(r ** 2)), 1e-30))
    if rel_rms is not None:
        assert rms < rel_rms, f"{what}: relative RMS error {rms:.2e}"
    return {"rel_rms": rms, "worst_over_bar": float((err / tol).max())}


# ---------------------------------------------------------------- bf16 experts

def run_bf16(lib, d, flags, seed, transpose_b=True, a_off=None, ids=None, usage=None):
    a_off = d.a_offsets if a_off is None else a_off
    ids = d.expert_ids if ids is None else ids
    usage = d.usage if usage is None else usage
    T, K = d.a.shape
    E, N, _ = d.b.shape
    n_out = N // 2 if flags & GATE else N
    bias, res = synth.grouped_epilogue_operands(seed, E, T, n_out, N, "bf16", std=0.02)
    b = d.b if transpose_b else np.ascontiguousarray(d.b.transpose(0, 2, 1))
    out = Guarded((T, n_out), torch.bfloat16, SENT["bf16"])
    lib.grouped_gemm_epilogue(out.view, dev16(d.a, torch.bfloat16), dev32(a_off), dev16(b, torch.bfloat16),
                              dev32(np.asarray(ids, np.int32)), [int(v) for v in usage], flags,
                              bias=dev16(bias, torch.bfloat16) if flags & BIAS else None,
                              residual=dev16(res, torch.bfloat16) if flags & RES else None,
                              transpose_b=transpose_b)
    got = host16(out.view)
    assert out.bands_intact(), "write outside C"
    c0 = np.full((T, n_out), SENT["bf16"], np.uint16)
    ref = oracle.grouped_gemm(c0, d.a, a_off, b, ids, usage, transpose_b=transpose_b, epilogue=flags,
                              bias_bits=bias, residual_bits=res)
    return compare(got, ref, SENT["bf16"], nm.decode_bf16, f"bf16 flags={flags} tb={transpose_b}", rel_rms=3e-3)


@pytest.mark.parametrize("flags", range(1, 8))
def test_bf16_every_flag_set(gpu, lib, flags):
    for (E, T, K, N, seed) in [(8, 200, 64, 64, 1), (5, 77, 40, 32, 2), (16, 600, 256, 208, 3)]:
        d = synth.grouped_inputs(seed=seed, E=E, T=T, K=K, N=N, skip_frac=0.25)
        say(f"[grouped-epi] bf16 flags={flags} E={E} T={T} K={K} N={N}")
        run_bf16(lib, d, flags, seed + 10 * flags)
        run_bf16(lib, d, flags, seed + 10 * flags, transpose_b=False)


# row-tile counts 1 .. 8 per tile (groups of 1 .. 128 rows) and K / N tails
@pytest.mark.parametrize("seed", [40, 41, 42])
def test_bf16_tile_heights(gpu, lib, seed):
    d = synth.grouped_inputs(seed=seed, E=6, T=500 + seed, K=128 + 8 * (seed - 40), N=144, skip_frac=0.2)
    say(f"[grouped-epi] bf16 seed {seed}")
    run_bf16(lib, d, BIAS | GATE | RES, seed)
    run_bf16(lib, d, BIAS | RES, seed + 1, transpose_b=False)


def test_bf16_edges_and_full_size(gpu, lib):
    d = synth.grouped_inputs(seed=8, E=4, T=200, K=64, N=64, skip_frac=0.0)
    a_off = np.array([5, 5, 60, 61, 150], np.uint32)
    ids = np.array([2, 2, 0, 3], np.int32)
    run_bf16(lib, d, 7, 1, a_off=a_off, ids=ids, usage=np.array([89, 4], np.uint32))
    run_bf16(lib, d, 5, 2, a_off=a_off, ids=ids, usage=np.array([89, 2], np.uint32))
    full = synth.grouped_inputs()
    say("[grouped-epi] bf16 full size, gated")
    say("  diagnostics", run_bf16(lib, full, 7, 3))


# ---------------------------------------------------------------- W4 experts

def run_w4(lib, d, flags, seed, a_off=None, ids=None, usage=None):
    """fp16 or bf16 (d.dtype). Gated outputs come from kernels that keep the 4-bit
    weights exact in their MFMAs (both types), so every output has the common bar."""
    a_off = d.a_offsets if a_off is None else a_off
    ids = d.expert_ids if ids is None else ids
    usage = d.usage if usage is None else usage
    T, K = d.a.shape
    E, _, N = d.b.shape
    n_out = N // 2 if flags & GATE else N
    bf16 = d.dtype == "bf16"
    tdt, sent, dec = (torch.bfloat16, SENT["bf16"], nm.decode_bf16) if bf16 else (torch.float16, SENT["f16"], nm.decode_f16)
    bias, res = synth.grouped_epilogue_operands(seed, E, T, n_out, N, d.dtype)
    out = Guarded((T, n_out), tdt, sent)
    lib.grouped_gemm_w4_epilogue(out.view, dev16(d.a, tdt), dev32(a_off), dev32(d.b),
                                 dev16(d.scales, tdt), dev32(np.asarray(ids, np.int32)),
                                 [int(v) for v in usage], flags,
                                 bias=dev16(bias, tdt) if flags & BIAS else None,
                                 residual=dev16(res, tdt) if flags & RES else None,
                                 group_size=d.group_size)
    got = host16(out.view)
    assert out.bands_intact(), "write outside C"
    c0 = np.full((T, n_out), sent, np.uint16)
    ref = oracle.grouped_gemm_w4(c0, d.a, a_off, d.b, d.scales, ids, usage, d.group_size, epilogue=flags,
                                 bias_bits=bias, residual_bits=res, dtype=d.dtype)
    return compare(got, ref, sent, dec, f"w4 {d.dtype} flags={flags}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("flags", range(1, 8))
def test_w4_every_flag_set(gpu, lib, flags, dtype):
    for (E, T, K, N, seed) in [(8, 200, 256, 64, 1), (5, 77, 128, 48, 2), (16, 600, 512, 208, 3)]:
        d = synth.grouped_w4_inputs(seed=seed, E=E, T=T, K=K, N=N, skip_frac=0.25, dtype=dtype)
        say(f"[grouped-epi] w4 {dtype} flags={flags} E={E} T={T} K={K} N={N}")
        run_w4(lib, d, flags, seed + 10 * flags)


@pytest.mark.parametrize("seed", [50, 51, 52])
def test_w4_ragged(gpu, lib, seed):
    d = synth.grouped_w4_inputs(seed=seed, E=6, T=500 + seed, K=256 - 32 * (seed - 50), N=144, skip_frac=0.2,
                                group_size=32)
    say(f"[grouped-epi] w4 seed {seed}")
    run_w4(lib, d, BIAS | GATE | RES, seed)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_w4_full_size(gpu, lib, dtype):
    d = synth.grouped_w4_inputs(dtype=dtype)
    say(f"[grouped-epi] w4 {dtype} full size, gated")
    say("  diagnostics", run_w4(lib, d, 7, 4))
    say("  diagnostics", run_w4(lib, d, BIAS | RES, 5))


def test_no_flags_match_the_plain_calls(gpu, lib):
    d = synth.grouped_inputs(seed=11, E=8, T=300, K=128, N=96, skip_frac=0.25)
    T, N = d.a.shape[0], d.b.shape[1]
    o1 = Guarded((T, N), torch.bfloat16, SENT["bf16"])
    o2 = Guarded((T, N), torch.bfloat16, SENT["bf16"])
    args = (dev16(d.a, torch.bfloat16), dev32(d.a_offsets), dev16(d.b, torch.bfloat16), dev32(d.expert_ids))
    lib.grouped_gemm(o1.view, *args, [int(v) for v in d.usage])
    lib.grouped_gemm_epilogue(o2.view, *args, [int(v) for v in d.usage], 0)
    assert np.array_equal(host16(o1.view), host16(o2.view))
