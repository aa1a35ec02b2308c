"""GPU parity of qgemm_w4_epilogue (through the C ABI) against the CPU oracle.

The Modular page "multistage_gemm_q" takes an optional function applied to each
output element (Parameters: elementwise_lambda_fn). The library offers three
fixed steps in its place: bias over columns, a SiLU-gated product of column
pairs (2j, 2j+1) that halves N, and a residual add, all on the fp32 product
before its one rounding.

Tolerance. Bias and residual outputs: the common bar |gpu - oracle| <=
1e-2 (|oracle| + 1) per element. A gated output z = silu(g) u amplifies the
GEMM's own error: with g ~ 8 and u ~ 0.2, the fp16 rounding of each weight
(q - 8) s alone moves z by more than 1e-2 (|z| + 1) (seen on the full-size
prefill, and reproduced on the CPU by rounding the weights to fp16 before an
exact product). So for gated outputs the common bar is put on the GEMM result
(tau_g = 1e-2 (|g| + 1), tau_u likewise) and carried through the gate to first
order with silu' in [-0.1, 1.1]: 1.1 |u| tau_g + (|silu(g)| + 1.1 tau_g) tau_u,
plus the common bar on z itself.
The bf16 prefill path rounds every weight to bf16 before the MFMAs; there the
bound follows from that arithmetic, per element:
  * Y's error: u_w = 2^-8 relative to |A| . |W| for the weight rounding, plus
    K * 2^-24 of fp32 accumulation slack;
  * the gate propagates it as above, plus fp32 rounding and exp error of a
    few ulps (2^-20 of |g u| and |z|);
  * both sides round to bf16 once: + 2 u_o |z| with u_o = 2^-8.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import REL, Guarded, dev16, dev32, host16, say

pytestmark = pytest.mark.gpu

SENT = {"f16": 0x7E00, "bf16": 0xFFC1}   # NaN patterns the kernels never write
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}
DEC = {"f16": oracle.numerics.decode_f16, "bf16": oracle.numerics.decode_bf16}
BIAS, RES, GATE = oracle.EPI_BIAS, oracle.EPI_RESIDUAL, oracle.EPI_SILU_GATE


def n_out(N, flags):
    return N // 2 if flags & GATE else N


def operands(w, flags, seed):
    M, N, _ = w.shape
    bias, res = synth.w4_epilogue_operands(seed, M, n_out(N, flags), N, w.dtype)
    return (bias if flags & BIAS else None), (res if flags & RES else None)


def run_epi(lib, w, flags, bias, res, env=None, variant=None):
    M, N, K = w.shape
    tdt = TDT[w.dtype]
    out = Guarded((M, n_out(N, flags)), tdt, SENT[w.dtype])
    if variant is not None:
        os.environ[env] = str(variant)
    try:
        lib.qgemm_w4_epilogue(out.view, dev16(w.a, tdt), dev32(w.b), dev16(w.scales, tdt), flags,
                              bias=dev16(bias, tdt) if bias is not None else None,
                              residual=dev16(res, tdt) if res is not None else None,
                              group_size=w.group_size)
    finally:
        if variant is not None:
            del os.environ[env]
    got = host16(out.view)
    assert out.bands_intact(), "write outside C"
    return got


def bound(w, flags, bias, res, rows=None):
    M, N, K = w.shape
    a_bits = w.a if rows is None else w.a[rows]
    dec = DEC[w.dtype]
    mag = np.abs(dec(a_bits)) @ np.abs(oracle.w4.dequant_w4(w.b, w.scales, w.group_size, dtype=w.dtype))
    y = oracle.w4.qgemm_w4_f64(a_bits, w.b, w.scales, w.group_size, dtype=w.dtype)
    prefill_bf16 = w.dtype == "bf16" and M > 16
    u_w = 2.0 ** -8 if prefill_bf16 else 2.0 ** -11
    e = (u_w + K * 2.0 ** -24) * mag
    if flags & BIAS:
        y = y + dec(bias)[None, :]
    e = e + 2.0 ** -20 * np.abs(y)
    if flags & GATE:
        g, u, eg, eu = y[:, 0::2], y[:, 1::2], e[:, 0::2], e[:, 1::2]
        z = oracle.silu(g) * u
        e = 1.1 * np.abs(u) * eg + (np.abs(oracle.silu(g)) + 1.1 * eg) * eu + 2.0 ** -20 * (np.abs(g * u) + np.abs(z))
    else:
        z = y
    if flags & RES:
        z = z + dec(res if rows is None else res[rows])
        e = e + 2.0 ** -22 * np.abs(z)
    u_o = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -11
    floor = 2.0 ** -24 if w.dtype == "f16" else 1e-30
    return e * (1 + u_o) + 2 * u_o * np.abs(z) + floor


def gate_tolerance(w, flags, bias, r, rows=None):
    """The common bar on the gate's inputs, carried through the gate, plus the bar on z."""
    a_bits = w.a if rows is None else w.a[rows]
    y = oracle.w4.qgemm_w4_f64(a_bits, w.b, w.scales, w.group_size, dtype=w.dtype)
    if flags & BIAS:
        y = y + DEC[w.dtype](bias)[None, :]
    g, u = y[:, 0::2], y[:, 1::2]
    tg, tu = REL * (np.abs(g) + 1.0), REL * (np.abs(u) + 1.0)
    return 1.1 * np.abs(u) * tg + (np.abs(oracle.silu(g)) + 1.1 * tg) * tu + REL * (np.abs(r) + 1.0)


def check(lib, w, flags, seed, what, rows=None, **kw):
    M, N, K = w.shape
    say(f"[w4-epi] {what}: M={M} N={N} K={K} gs={w.group_size} {w.dtype} flags={flags} {kw}")
    bias, res = operands(w, flags, seed)
    got = run_epi(lib, w, flags, bias, res, **kw)
    if rows is not None:
        got = got[rows]
    ref = oracle.qgemm_w4_epilogue(w.a if rows is None else w.a[rows], w.b, w.scales, w.group_size, flags,
                                   bias, None if res is None else (res if rows is None else res[rows]),
                                   dtype=w.dtype)
    dec = DEC[w.dtype]
    g, r = dec(got), dec(ref)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    if w.dtype == "bf16" and M > 16:
        b = bound(w, flags, bias, res, rows)
    elif flags & GATE:
        b = gate_tolerance(w, flags, bias, r, rows)
    else:
        b = REL * (np.abs(r) + 1.0)
    err = np.abs(g - r)
    bad = err > b
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond the tolerance, first "
                           f"{np.argwhere(bad)[:3].tolist()}, worst {float((err / b).max()):.3f} x bound")
    return float((err / b).max())


DECODE_SHAPES = [(16, 256, 512, 128), (3, 272, 384, 128), (1, 16, 256, 32), (7, 528, 512, 64), (2, 192, 2048, 256)]
PREFILL_SHAPES = [(48, 256, 512, 128), (17, 16, 256, 128), (100, 144, 96, 32), (257, 1008, 448, 64)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("flags", range(8))
def test_every_flag_set_default_paths(gpu, lib, flags, dtype):
    for i, (M, N, K, gs) in enumerate(DECODE_SHAPES + PREFILL_SHAPES):
        w = synth.w4_inputs(M, N, K, seed=M + N + flags, group_size=gs, dtype=dtype)
        check(lib, w, flags, 1000 + i, "default")


@pytest.mark.parametrize("variant", range(9, 16))
def test_decode_variants(gpu, lib, variant):
    for flags in (BIAS, RES, GATE, BIAS | GATE | RES):
        for dtype in ("f16", "bf16"):
            for (M, N, K, gs) in DECODE_SHAPES[:3]:
                w = synth.w4_inputs(M, N, K, seed=3 * M + N, group_size=gs, dtype=dtype)
                check(lib, w, flags, 7 + flags, f"decode v{variant}", env="QG_W4_DECODE_VARIANT", variant=variant)


@pytest.mark.parametrize("variant", range(11, 20))
def test_prefill_variants(gpu, lib, variant):
    for flags in (BIAS, RES, GATE, BIAS | GATE | RES):
        for dtype in ("f16", "bf16"):
            for (M, N, K, gs) in PREFILL_SHAPES[:3]:
                w = synth.w4_inputs(M, N, K, seed=M + 5 * N, group_size=gs, dtype=dtype)
                check(lib, w, flags, 9 + flags, f"prefill v{variant}", env="QG_W4_PREFILL_VARIANT",
                      variant=variant)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_full_size(gpu, lib, dtype):
    """Decode M = 1, 16 at N = K = 4096 and the 2048 x 11008 x 4096 prefill (48
    sampled rows), with bias and residual, ungated and gated (output N / 2)."""
    for flags in (BIAS | RES, BIAS | GATE | RES):
        for c in synth.W4_DECODE:
            if c["M"] in (1, 16):
                check(lib, synth.w4_inputs(**c, dtype=dtype), flags, 21, "decode full")
        w = synth.w4_inputs(**synth.W4_PREFILL, dtype=dtype)
        M = w.shape[0]
        rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(2).choice(M, 48, replace=False)]))
        d = check(lib, w, flags, 22, "prefill full", rows=rows)
        say("  worst error / tolerance", d)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_no_flags_is_qgemm_w4(gpu, lib, dtype):
    """Epilogue 0 returns exactly qgemm_w4's bits (decode and prefill)."""
    for (M, N, K, gs) in [(5, 512, 1024, 128), (300, 1024, 1024, 128)]:
        w = synth.w4_inputs(M, N, K, seed=M, group_size=gs, dtype=dtype)
        tdt = TDT[dtype]
        plain = torch.empty((M, N), dtype=tdt, device="cuda")
        lib.qgemm_w4(plain, dev16(w.a, tdt), dev32(w.b), dev16(w.scales, tdt), gs)
        assert np.array_equal(run_epi(lib, w, 0, None, None), host16(plain))


def test_zero_activations_give_bias_and_residual_exactly(gpu, lib):
    """A = 0: Y = 0, so bias alone, residual alone and the gated residual
    (silu(0) * 0 + r) come back bit-exact."""
    for M in (4, 64):
        w = synth.w4_inputs(M, 256, 512, seed=8)
        w.a[:] = 0
        bias, res = synth.w4_epilogue_operands(3, M, 256, 256)
        assert np.array_equal(run_epi(lib, w, BIAS, bias, None), np.broadcast_to(bias, (M, 256)))
        assert np.array_equal(run_epi(lib, w, RES, None, res), res)
        _, res2 = synth.w4_epilogue_operands(4, M, 128, 256)
        assert np.array_equal(run_epi(lib, w, GATE | RES, None, res2), res2)


def test_determinism(gpu, lib):
    w = synth.w4_inputs(300, 1024, 1024, seed=12)
    bias, res = operands(w, 7, 5)
    assert np.array_equal(run_epi(lib, w, 7, bias, res), run_epi(lib, w, 7, bias, res))
