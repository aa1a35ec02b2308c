"""GPU parity of grouped_gemm (through the C ABI) against the CPU oracle.

Modular page "grouped_matmul_sm100_persistent": a_offsets prefix sum,
expert_ids with negative entries skipped, expert_usage_stats[1] active count.
Floats: |gpu - oracle| <= 1e-2 (|oracle| + 1); routing (which rows are written,
which expert each used) bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, assert_close, bf16v, dev16, dev32, host16, say
from oracle import numerics as nm

pytestmark = pytest.mark.gpu

SENT = 0xFFC1  # bf16 NaN pattern: never produced by the kernel


def run_grouped(lib, d: synth.GroupedInputs, a_off=None, ids=None, usage=None, transpose_b=True):
    a_off = d.a_offsets if a_off is None else a_off
    ids = d.expert_ids if ids is None else ids
    usage = d.usage if usage is None else usage
    T, K = d.a.shape
    N = d.b.shape[1]
    # transpose_b == False: the same expert matrices stored [E, K, N]
    b = d.b if transpose_b else np.ascontiguousarray(d.b.transpose(0, 2, 1))
    out = Guarded((T, N), torch.bfloat16, SENT)
    lib.grouped_gemm(out.view, dev16(d.a, torch.bfloat16), dev32(a_off), dev16(b, torch.bfloat16),
                     dev32(np.asarray(ids, np.int32)), [int(v) for v in usage], transpose_b)
    got = host16(out.view)
    assert out.bands_intact(), "write outside C"
    return got


def check(lib, d, what, **kw):
    T, K = d.a.shape
    say(f"[grouped] {what}: T={T} K={K} N={d.b.shape[1]} E={d.b.shape[0]}")
    got = run_grouped(lib, d, **kw)
    a_off = kw.get("a_off", d.a_offsets)
    ids = kw.get("ids", d.expert_ids)
    usage = kw.get("usage", d.usage)
    c0 = np.full(got.shape, SENT, np.uint16)
    if kw.get("transpose_b", True):
        ref = oracle.grouped_gemm(c0, d.a, a_off, d.b, ids, usage)
    else:
        ref = oracle.grouped_gemm(c0, d.a, a_off, np.ascontiguousarray(d.b.transpose(0, 2, 1)), ids, usage,
                                  transpose_b=False)
    written = ref[:, 0] != SENT
    # routing: exactly the rows the oracle writes are written
    assert np.array_equal(got[:, 0] != SENT, written), "row routing differs"
    assert np.all(got[~written] == SENT)
    if written.any():
        return assert_close(bf16v(got[written]), bf16v(ref[written]), what=what)
    return {}


def test_small_ragged(gpu, lib):
    for (E, T, K, N, seed) in [(8, 200, 64, 64, 1), (5, 77, 40, 24, 2), (16, 600, 256, 200, 3), (3, 300, 96, 136, 4)]:
        d = synth.grouped_inputs(seed=seed, E=E, T=T, K=K, N=N, skip_frac=0.25)
        check(lib, d, f"small seed{seed}")


def test_large_groups_span_row_blocks(gpu, lib):
    """Groups with more than 128 rows are split into several row blocks."""
    d = synth.grouped_inputs(seed=7, E=3, T=900, K=128, N=72, skip_frac=0.0)
    check(lib, d, "large groups")


def test_edges_empty_duplicate_partial(gpu, lib):
    d = synth.grouped_inputs(seed=8, E=4, T=200, K=64, N=64, skip_frac=0.0)
    a_off = np.array([5, 5, 60, 61, 150], np.uint32)       # empty group 0; rows 0..4 and 150.. unlisted
    ids = np.array([2, 2, 0, 3], np.int32)                   # expert 2 twice
    check(lib, d, "edges", a_off=a_off, ids=ids, usage=np.array([89, 4], np.uint32))
    check(lib, d, "partial active", a_off=a_off, ids=ids, usage=np.array([89, 2], np.uint32))


def test_skip_everything(gpu, lib):
    d = synth.grouped_inputs(seed=9, E=4, T=64, K=64, N=64)
    got = run_grouped(lib, d, ids=np.full(4, -1, np.int32))
    assert np.all(got == SENT)


def test_routing_scaled_identity_bit_exact(gpu, lib):
    """B[e] = 2^((e mod 16) - 8) I: every written row is its A row times its expert's factor, exactly."""
    E, T, K = 20, 700, 64
    d = synth.grouped_inputs(seed=10, E=E, T=T, K=K, N=K, skip_frac=0.2)
    ids = np.random.default_rng(1).permutation(d.expert_ids).astype(np.int32)
    fac = np.ldexp(1.0, (np.arange(E) % 16) - 8)
    d.b = nm.bf16_bits_of(fac[:, None, None] * np.eye(K)[None])
    got = run_grouped(lib, d, ids=ids)
    a = bf16v(d.a)
    for g in range(E):
        r0, r1 = d.a_offsets[g], d.a_offsets[g + 1]
        if ids[g] < 0:
            assert np.all(got[r0:r1] == SENT)
        else:
            assert np.array_equal(bf16v(got[r0:r1]), a[r0:r1] * fac[ids[g]]), g


def test_full_size_config(gpu, lib):
    """64 experts, 4096 routed rows, K=2048, N=1408, 10% skipped: every element checked."""
    d = synth.grouped_inputs()
    diag = check(lib, d, "full")
    say("  diagnostics", diag)
    assert diag["rel_rms"] < 3e-3


def test_determinism(gpu, lib):
    d = synth.grouped_inputs(seed=11, E=16, T=1000, K=256, N=192)
    assert np.array_equal(run_grouped(lib, d), run_grouped(lib, d))


# ragged shapes: K tails (K % 32 != 0), N tails, tiny and large groups, 25% skipped
GROUPED_SHAPES = [(8, 200, 64, 64, 21), (5, 77, 40, 24, 22), (16, 600, 456, 200, 23), (3, 300, 96, 136, 24),
                  (4, 520, 384, 72, 25), (6, 900, 136, 48, 26), (4, 520, 72, 1032, 15)]


@pytest.mark.parametrize("transpose_b", [True, False], ids=["ENK", "EKN"])
@pytest.mark.parametrize("shape", GROUPED_SHAPES, ids=lambda s: f"E{s[0]}_T{s[1]}_K{s[2]}_N{s[3]}")
def test_ragged_shapes(gpu, lib, shape, transpose_b):
    E, T, K, N, seed = shape
    d = synth.grouped_inputs(seed=seed, E=E, T=T, K=K, N=N, skip_frac=0.25)
    check(lib, d, f"seed{seed} tb={transpose_b}", transpose_b=transpose_b)


def test_b_not_transposed_full_size(gpu, lib):
    """64 experts, 4096 routed rows, K = 2048, N = 1408, experts stored [E, K, N]."""
    d = synth.grouped_inputs()
    diag = check(lib, d, "full [E,K,N]", transpose_b=False)
    say("  diagnostics", diag)
