"""Pins for the grouped GEMM oracle (Modular page
"grouped_matmul_sm100_persistent": a_offsets prefix sum, expert_ids with
negative entries skipping, expert_usage_stats[1] = active count, transpose_b)."""
import json
import os

import numpy as np
import torch

import oracle
from oracle import numerics as nm
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "grouped_worked_example.json")
SENT = 0xFFC1  # a bf16 NaN pattern used as "never written" sentinel


def test_worked_example_from_fixture():
    g = json.load(open(GOLD))
    a = nm.bf16_bits_of(np.array(g["A"], dtype=np.float64))
    b = nm.bf16_bits_of(np.array(g["B"], dtype=np.float64))
    c0 = nm.bf16_bits_of(np.array(g["C_prior"], dtype=np.float64))
    c = oracle.grouped_gemm(c0, a, np.array(g["a_offsets"], np.uint32), b,
                            np.array(g["expert_ids"], np.int32), np.array(g["usage"], np.uint32))
    assert np.array_equal(nm.decode_bf16(c), np.array(g["C_expected"], dtype=np.float64))


def test_single_group_reduces_to_plain_gemm():
    T, K, N = 37, 64, 24
    d = synth.grouped_inputs(seed=1, E=1, T=T, K=K, N=N, skip_frac=0.0)
    c0 = np.full((T, N), SENT, np.uint16)
    c = oracle.grouped_gemm(c0, d.a, np.array([0, T], np.uint32), d.b, np.array([0], np.int32),
                            np.array([T, 1], np.uint32))
    ta = torch.from_numpy(nm.decode_bf16(d.a))
    tb = torch.from_numpy(nm.decode_bf16(d.b[0]))
    ref = (ta @ tb.T).numpy()
    assert np.array_equal(nm.decode_bf16(c), nm.round_to_bf16(ref))


def test_skip_everything_leaves_c_untouched():
    d = synth.grouped_inputs(seed=2, E=4, T=20, K=32, N=16)
    c0 = np.full((20, 16), SENT, np.uint16)
    ids = np.full(4, -1, np.int32)
    assert np.array_equal(oracle.grouped_gemm(c0, d.a, d.a_offsets, d.b, ids, d.usage), c0)
    assert np.array_equal(oracle.grouped_gemm(c0, d.a, d.a_offsets, d.b, d.expert_ids,
                                              np.array([5, 0], np.uint32)), c0)


def test_routing_with_scaled_identities_is_exact():
    """B[e] = 2^((e mod 16) - 8) * I, so each written row is its A row times its expert's factor."""
    E, T, K = 12, 90, 32
    rng = np.random.default_rng(3)
    d = synth.grouped_inputs(seed=3, E=E, T=T, K=K, N=K, skip_frac=0.2)
    ids = rng.permutation(d.expert_ids)
    fac = np.ldexp(1.0, (np.arange(E) % 16) - 8)
    b = nm.bf16_bits_of(fac[:, None, None] * np.eye(K)[None])
    c0 = np.full((T, K), SENT, np.uint16)
    c = oracle.grouped_gemm(c0, d.a, d.a_offsets, b, ids, d.usage)
    a = nm.decode_bf16(d.a)
    for g in range(E):
        r0, r1 = d.a_offsets[g], d.a_offsets[g + 1]
        if ids[g] < 0:
            assert np.all(c[r0:r1] == SENT)
        else:
            assert np.array_equal(nm.decode_bf16(c[r0:r1]), a[r0:r1] * fac[ids[g]])


def test_edges_empty_duplicate_partial_offset():
    """Empty groups, repeated experts, fewer active groups than listed, a_offsets[0] > 0."""
    T, K, N = 30, 16, 8
    d = synth.grouped_inputs(seed=4, E=3, T=T, K=K, N=N, skip_frac=0.0)
    a_off = np.array([2, 2, 9, 20, 28], np.uint32)       # group 0 empty; rows 0..1, 28.. unlisted
    ids = np.array([1, 1, 0, 2], np.int32)                # expert 1 twice
    usage = np.array([11, 3], np.uint32)                  # group 3 not active
    c0 = np.full((T, N), SENT, np.uint16)
    c = oracle.grouped_gemm(c0, d.a, a_off, d.b, ids, usage)
    a = nm.decode_bf16(d.a)
    b = nm.decode_bf16(d.b)
    assert np.all(c[:2] == SENT) and np.all(c[20:] == SENT)
    assert np.array_equal(nm.decode_bf16(c[2:9]), nm.round_to_bf16(a[2:9] @ b[1].T))
    assert np.array_equal(nm.decode_bf16(c[9:20]), nm.round_to_bf16(a[9:20] @ b[0].T))


def test_brute_force_loops_and_both_b_layouts():
    E, G, T, K, N = 4, 5, 40, 32, 32
    rng = np.random.default_rng(5)
    d = synth.grouped_inputs(seed=5, E=E, T=T, K=K, N=N, skip_frac=0.0)
    cuts = np.sort(rng.integers(0, T + 1, G - 1))
    a_off = np.concatenate([[0], cuts, [T]]).astype(np.uint32)
    ids = np.array([3, -1, 0, 3, 1], np.int32)
    usage = np.array([T, G], np.uint32)
    c0 = np.full((T, N), SENT, np.uint16)
    c = oracle.grouped_gemm(c0, d.a, a_off, d.b, ids, usage)
    a = nm.decode_bf16(d.a)
    b = nm.decode_bf16(d.b)
    ref = np.full((T, N), np.nan)
    for g in range(G):
        if ids[g] < 0:
            continue
        for r in range(a_off[g], a_off[g + 1]):
            for n in range(N):
                ref[r, n] = sum(a[r, k] * b[ids[g], n, k] for k in range(K))
    written = ~np.isnan(ref[:, 0])
    assert np.array_equal(nm.decode_bf16(c[written]), nm.round_to_bf16(ref[written]))
    assert np.all(c[~written] == SENT)
    # transpose_b = False: the same weights stored [E, K, N]
    bt = np.ascontiguousarray(d.b.transpose(0, 2, 1))
    c2 = oracle.grouped_gemm(c0, d.a, a_off, bt, ids, usage, transpose_b=False)
    assert np.array_equal(c2, c)


# ---------------------------------------------------------------- fixed epilogues

def _sig(x):
    import math
    return 0.5 * (1.0 + math.tanh(0.5 * x))


def test_epilogue_brute_force_loops():
    """Bias row of the group's expert, SiLU-gated column pairs, residual, one rounding."""
    E, G, T, K, N = 4, 5, 30, 32, 32
    rng = np.random.default_rng(6)
    d = synth.grouped_inputs(seed=6, E=E, T=T, K=K, N=N, skip_frac=0.0)
    cuts = np.sort(rng.integers(0, T + 1, G - 1))
    a_off = np.concatenate([[0], cuts, [T]]).astype(np.uint32)
    ids = np.array([3, -1, 0, 3, 1], np.int32)
    usage = np.array([T, G], np.uint32)
    a, b = nm.decode_bf16(d.a), nm.decode_bf16(d.b)
    for flags in range(8):
        n_out = N // 2 if flags & oracle.EPI_SILU_GATE else N
        bias, res = synth.grouped_epilogue_operands(flags, E, T, n_out, N, std=0.02)
        c0 = np.full((T, n_out), SENT, np.uint16)
        c = oracle.grouped_gemm(c0, d.a, a_off, d.b, ids, usage, epilogue=flags, bias_bits=bias, residual_bits=res)
        bf, rf = nm.decode_bf16(bias), nm.decode_bf16(res)
        for g in range(G):
            for r in range(a_off[g], a_off[g + 1]):
                if ids[g] < 0:
                    assert np.all(c[r] == SENT)
                    continue
                y = [sum(a[r, k] * b[ids[g], n, k] for k in range(K)) for n in range(N)]
                if flags & oracle.EPI_BIAS:
                    y = [y[n] + bf[ids[g], n] for n in range(N)]
                z = [y[2 * j] * _sig(y[2 * j]) * y[2 * j + 1] for j in range(N // 2)] \
                    if flags & oracle.EPI_SILU_GATE else y
                if flags & oracle.EPI_RESIDUAL:
                    z = [z[j] + rf[r, j] for j in range(n_out)]
                got = nm.decode_bf16(c[r])
                exact = np.array(z)
                ulp = np.abs(nm.round_to_bf16(exact * (1 + 2.0 ** -7)) - nm.round_to_bf16(exact)) + 1e-40
                assert np.all(np.abs(got - exact) <= ulp), (flags, g, r)


def test_epilogue_bias_row_is_the_groups_expert():
    """A = 0: every written row is its group's expert's bias row, exactly."""
    E, T, K, N = 4, 12, 32, 16
    d = synth.grouped_inputs(seed=7, E=E, T=T, K=K, N=N, skip_frac=0.0)
    a = np.zeros_like(d.a)
    a_off = np.array([0, 3, 5, 9, 12], np.uint32)
    ids = np.array([2, -1, 0, 2], np.int32)
    bias, _ = synth.grouped_epilogue_operands(1, E, T, N, N)
    c0 = np.full((T, N), SENT, np.uint16)
    c = oracle.grouped_gemm(c0, a, a_off, d.b, ids, np.array([4, 4], np.uint32), epilogue=oracle.EPI_BIAS,
                            bias_bits=bias)
    for g, e in enumerate(ids):
        rows = slice(a_off[g], a_off[g + 1])
        assert np.all(c[rows] == (SENT if e < 0 else bias[e])), g


# ---------------------------------------------------------------- a_plane_splits (fused LoRA QKV planes)

GOLD_PLANES = os.path.join(os.path.dirname(__file__), "golden", "grouped_planes_worked_example.json")


def _bits(x):
    return nm.bf16_bits_of(np.asarray(x, dtype=np.float64))


def test_planes_worked_example_from_fixture():
    g = json.load(open(GOLD_PLANES))
    c = oracle.grouped_gemm(_bits(g["C_prior"]), _bits(g["A"]), np.array(g["a_offsets"], np.uint32), _bits(g["B"]),
                            np.array(g["expert_ids"], np.int32), np.array(g["usage"], np.uint32),
                            a_plane_splits=g["a_plane_splits"])
    assert np.array_equal(nm.decode_bf16(c), np.array(g["C_expected"], dtype=np.float64))


def test_planes_off_is_the_plain_product():
    d = synth.grouped_inputs(seed=30, E=5, T=70, K=48, N=40, skip_frac=0.2)
    c0 = np.full((70, 40), SENT, np.uint16)
    plain = oracle.grouped_gemm(c0, d.a, d.a_offsets, d.b, d.expert_ids, d.usage)
    assert np.array_equal(oracle.grouped_gemm(c0, d.a, d.a_offsets, d.b, d.expert_ids, d.usage,
                                              a_plane_splits=(0, 0)), plain)


def _plane_of(n, s0, s1):
    return 0 if n < s0 else (1 if n < s0 + s1 else 2)


def test_planes_route_columns_exactly():
    """B[e] = c_e I and plane p of A = (p + 1) X: column n of row r is c_e (p(n) + 1) X[r, n],
    exact in bf16 (power-of-two factors and small integers), for both B layouts and
    splits that include an empty plane."""
    E, T, K = 4, 40, 48
    rng = np.random.default_rng(31)
    x = rng.integers(-8, 9, size=(T, K)).astype(np.float64)
    a = _bits(np.concatenate([x, 2 * x, 3 * x]))
    fac = np.ldexp(1.0, np.arange(E) - 2)
    b = _bits(fac[:, None, None] * np.eye(K)[None])
    a_off = np.array([0, 7, 7, 30, 40], np.uint32)
    ids = np.array([2, 0, -1, 3], np.int32)
    for s0, s1 in [(16, 8), (0, 24), (48, 0), (5, 40)]:
        for tb in (True, False):
            c = oracle.grouped_gemm(np.full((T, K), SENT, np.uint16), a, a_off, b, ids, [23, 4], transpose_b=tb,
                                    a_plane_splits=(s0, s1))
            got = nm.decode_bf16(c)
            for g in range(4):
                r0, r1 = int(a_off[g]), int(a_off[g + 1])
                if ids[g] < 0:
                    assert np.all(c[r0:r1] == SENT)
                    continue
                for n in range(K):
                    want = fac[ids[g]] * (_plane_of(n, s0, s1) + 1) * x[r0:r1, n]
                    assert np.array_equal(got[r0:r1, n], want), (s0, s1, tb, g, n)


def test_planes_brute_force_integers():
    """Scalar loops over rows, columns and K with the plane looked up per column; small
    integer operands keep every sum exact, so the results agree bit for bit."""
    rng = np.random.default_rng(32)
    E, T, K, N = 3, 11, 5, 9
    a = rng.integers(-4, 5, size=(3 * T, K)).astype(np.float64)
    b = rng.integers(-4, 5, size=(E, N, K)).astype(np.float64)
    a_off = np.array([0, 4, 4, 9, 11], np.uint32)
    ids = np.array([1, 2, 0, -1], np.int32)
    s0, s1 = 2, 4
    c = oracle.grouped_gemm(np.full((T, N), SENT, np.uint16), _bits(a), a_off, _bits(b), ids, [5, 4],
                            a_plane_splits=(s0, s1))
    want = np.full((T, N), np.nan)
    for g in range(4):
        if ids[g] < 0:
            continue
        for r in range(int(a_off[g]), int(a_off[g + 1])):
            for n in range(N):
                p = _plane_of(n, s0, s1)
                want[r, n] = sum(a[p * T + r, k] * b[ids[g], n, k] for k in range(K))
    written = ~np.isnan(want)
    assert np.array_equal(nm.decode_bf16(c)[written], want[written])
    assert np.all(c[~written] == SENT)


def test_planes_reject_bad_shapes():
    d = synth.grouped_inputs(seed=33, E=2, T=10, K=16, N=16)
    c0 = np.full((10, 16), SENT, np.uint16)
    import pytest
    with pytest.raises(ValueError):   # A must hold three planes
        oracle.grouped_gemm(c0, d.a, d.a_offsets, d.b, d.expert_ids, d.usage, a_plane_splits=(8, 4))
    a3 = np.concatenate([d.a, d.a, d.a])
    with pytest.raises(ValueError):   # splits beyond N
        oracle.grouped_gemm(c0, a3, d.a_offsets, d.b, d.expert_ids, d.usage, a_plane_splits=(12, 8))
