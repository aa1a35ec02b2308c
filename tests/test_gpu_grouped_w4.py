"""GPU parity of grouped_gemm_w4 (through the C ABI) against the CPU oracle.

The routing of the Modular page "grouped_matmul_sm100_persistent" (a_offsets
prefix sum, expert_ids with negative entries skipped, expert_usage_stats[1]
active count) over experts in the packed 4-bit format of "multistage_gemm_q"
(group_size, pack_factor), with fp16 or bf16 activations, scales and output.
Floats: |gpu - oracle| <= 1e-2 (|oracle| + 1); routing (which rows are written)
and unpacked weights: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, assert_close, bf16v, dev16, dev32, f16v, host16, say
from oracle import numerics as nm

pytestmark = pytest.mark.gpu

SENT = 0x7E00       # fp16 NaN pattern: never produced by the kernel
SENT_BF16 = 0xFFC1  # bf16 NaN pattern
DTYPES = ["f16", "bf16"]


def _sent(d):
    return SENT_BF16 if d.dtype == "bf16" else SENT


def run_gw4(lib, d, a_off=None, ids=None, usage=None, a=None):
    a_off = d.a_offsets if a_off is None else a_off
    ids = d.expert_ids if ids is None else ids
    usage = d.usage if usage is None else usage
    a = d.a if a is None else a
    T = a.shape[0]
    N = d.b.shape[2]
    tdt = torch.bfloat16 if d.dtype == "bf16" else torch.float16
    out = Guarded((T, N), tdt, _sent(d))
    lib.grouped_gemm_w4(out.view, dev16(a, tdt), dev32(a_off), dev32(d.b),
                        dev16(d.scales, tdt), dev32(np.asarray(ids, np.int32)),
                        [int(v) for v in usage], d.group_size)
    got = host16(out.view)
    assert out.bands_intact(), "write outside C"
    return got


def check(lib, d, what, **kw):
    a = kw.get("a", d.a)
    say(f"[grouped_w4] {what}: T={a.shape[0]} K={a.shape[1]} N={d.b.shape[2]} E={d.b.shape[0]} "
        f"gs={d.group_size} {d.dtype}")
    got = run_gw4(lib, d, **kw)
    a_off = kw.get("a_off", d.a_offsets)
    ids = kw.get("ids", d.expert_ids)
    usage = kw.get("usage", d.usage)
    sent = _sent(d)
    c0 = np.full(got.shape, sent, np.uint16)
    ref = oracle.grouped_gemm_w4(c0, a, a_off, d.b, d.scales, ids, usage, d.group_size, dtype=d.dtype)
    written = ref[:, 0] != sent
    assert np.array_equal(got[:, 0] != sent, written), "row routing differs"
    assert np.all(got[~written] == sent)
    v = bf16v if d.dtype == "bf16" else f16v
    if written.any():
        return assert_close(v(got[written]), v(ref[written]), what=what)
    return {}


@pytest.mark.parametrize("dtype", DTYPES)
def test_small_ragged(gpu, lib, dtype):
    for (E, T, K, N, gs, seed) in [(8, 200, 256, 64, 128, 1), (5, 77, 128, 24, 32, 2),
                                   (16, 600, 512, 264, 64, 3), (3, 300, 256, 136, 256, 4),
                                   (6, 150, 96, 40, 32, 5), (4, 90, 160, 48, 32, 6)]:   # K % 64 == 32: partial last stage
        d = synth.grouped_w4_inputs(seed=seed, E=E, T=T, K=K, N=N, skip_frac=0.25, group_size=gs, dtype=dtype)
        check(lib, d, f"small seed{seed}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_large_groups_and_edges(gpu, lib, dtype):
    """Groups of 0, 1, 127, 128, 129 and 300 rows; a_offsets[0] > 0; a repeated
    expert; num_active below the table length (the last group is not processed)."""
    d = synth.grouped_w4_inputs(seed=7, E=4, T=700, K=256, N=72, dtype=dtype)
    a_off = np.array([5, 5, 6, 133, 261, 390, 690, 700], np.uint32)
    ids = np.array([1, 0, 2, -1, 3, 1, 2], np.int32)
    check(lib, d, "edges", a_off=a_off, ids=ids, usage=np.array([300, 6], np.uint32))


@pytest.mark.parametrize("dtype", DTYPES)
def test_all_skipped_is_untouched(gpu, lib, dtype):
    d = synth.grouped_w4_inputs(seed=8, E=4, T=100, K=128, N=32, dtype=dtype)
    got = run_gw4(lib, d, ids=np.full(len(d.expert_ids), -1, np.int32))
    assert np.all(got == _sent(d))


@pytest.mark.parametrize("dtype", DTYPES)
def test_unit_rows_give_unpacked_weights_exactly(gpu, lib, dtype):
    """Row r of A is the unit vector e_{k_r}: C[r][n] = round((q - 8) * s) of the
    routed expert, compared bitwise."""
    E, T, K, N = 3, 96, 512, 80
    d = synth.grouped_w4_inputs(seed=9, E=E, T=T, K=K, N=N, dtype=dtype)
    rng = np.random.default_rng(9)
    ks = rng.integers(0, K, size=T)
    a = np.zeros((T, K), np.uint16)
    a[np.arange(T), ks] = 0x3F80 if dtype == "bf16" else 0x3C00
    a_off = np.array([0, 30, 31, 80, 96], np.uint32)
    ids = np.array([2, 0, -1, 1], np.int32)
    got = run_gw4(lib, d, a_off=a_off, ids=ids, usage=np.array([49, 4], np.uint32), a=a)
    ref = oracle.grouped_gemm_w4(np.full((T, N), _sent(d), np.uint16), a, a_off, d.b, d.scales, ids,
                                 np.array([49, 4], np.uint32), d.group_size, dtype=dtype)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dtype", DTYPES)
def test_full_size_config(gpu, lib, dtype):
    """64 int4 experts, 4096 routed rows (multinomial), K = 2048, N = 1408, 10% skipped."""
    d = synth.grouped_w4_inputs(dtype=dtype)
    diag = check(lib, d, "full")
    say("  diagnostics", diag)


@pytest.mark.parametrize("dtype", DTYPES)
def test_determinism(gpu, lib, dtype):
    d = synth.grouped_w4_inputs(seed=10, E=8, T=500, K=512, N=256, dtype=dtype)
    assert np.array_equal(run_gw4(lib, d), run_gw4(lib, d))
