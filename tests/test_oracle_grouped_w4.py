"""Pins for the grouped W4A16 oracle (no GPU).

The grouped W4A16 GEMM joins the routing of the Modular page
"grouped_matmul_sm100_persistent" (Args: a_offsets, expert_ids, negative ids
skip, expert_usage_stats[1]) with the packed weights of "multistage_gemm_q"
(Parameters: pack_factor, group_size). Pins:
  * one group over all rows reduces to the plain W4A16 oracle, bit for bit;
  * skipped and unprocessed groups leave C untouched;
  * a brute-force evaluation with its own bit extraction (Python integers) and
    numpy's own fp16 rounding agrees on tiny random problems;
  * experts built so each yields a different exact constant prove which expert
    every group used."""
import numpy as np

import oracle
import synth
from oracle import numerics as nm

SENT = 0x7E00


def _tiny(seed, E=3, G=4, T=20, K=64, N=16, gs=32):
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(T, [1.0 / G] * G)
    off = np.zeros(G + 1, np.uint32)
    off[1:] = np.cumsum(counts)
    ids = rng.integers(-1, E, size=G).astype(np.int32)
    a = synth.f16_bits(rng.standard_normal((T, K)))
    b = rng.integers(0, 2**32, size=(E, K // 8, N), dtype=np.uint32)
    s = synth.f16_bits(rng.uniform(0.005, 0.02, size=(E, K // gs, N)))
    return a, off, b, s, ids, gs


def test_single_group_reduces_to_w4():
    w = synth.w4_inputs(24, 40, 256, seed=11, group_size=64)
    T, N = w.a.shape[0], w.b.shape[1]
    got = oracle.grouped_gemm_w4(np.full((T, N), SENT, np.uint16), w.a, np.array([0, T], np.uint32),
                                 w.b[None], w.scales[None], np.array([0], np.int32), np.array([T, 1], np.uint32), 64)
    assert np.array_equal(got, oracle.qgemm_w4(w.a, w.b, w.scales, 64))


def test_skip_semantics():
    a, off, b, s, ids, gs = _tiny(1)
    c0 = np.full((a.shape[0], b.shape[2]), SENT, np.uint16)
    got = oracle.grouped_gemm_w4(c0, a, off, b, s, np.full_like(ids, -1), np.array([9, 4], np.uint32), gs)
    assert np.array_equal(got, c0)
    got = oracle.grouped_gemm_w4(c0, a, off, b, s, ids, np.array([9, 0], np.uint32), gs)
    assert np.array_equal(got, c0)


def test_brute_force_tiny():
    """Scalar loops with their own nibble extraction; numpy's float64 -> float16
    cast rounds. The two sums differ only in fp64 summation order, so a
    mismatch is allowed only where the exact value sits on an fp16 tie."""
    for seed in range(4):
        a, off, b, s, ids, gs = _tiny(seed)
        T, N, K = a.shape[0], b.shape[2], a.shape[1]
        c0 = np.full((T, N), SENT, np.uint16)
        usage = np.array([0, len(ids) - (seed % 2)], np.uint32)   # odd seeds drop the last group
        got = oracle.grouped_gemm_w4(c0, a, off, b, s, ids, usage, gs)
        av = a.view(np.float16).astype(np.float64)
        sv = s.view(np.float16).astype(np.float64)
        want = c0.copy()
        exact = np.zeros((T, N))
        for g in range(int(usage[1])):
            e = int(ids[g])
            if e < 0:
                continue
            for r in range(int(off[g]), int(off[g + 1])):
                for n in range(N):
                    acc = 0.0
                    for k in range(K):
                        q = (int(b[e, k // 8, n]) >> (4 * (k % 8))) & 0xF
                        acc += av[r, k] * (q - 8) * sv[e, k // gs, n]
                    exact[r, n] = acc
                    want[r, n] = np.float16(acc).view(np.uint16)
        for r, n in np.argwhere(got != want):
            lo, hi = sorted([float(got[r, n:n + 1].view(np.float16)[0]), float(want[r, n:n + 1].view(np.float16)[0])])
            assert abs(exact[r, n] - (lo + hi) / 2) <= 1e-12 * abs(exact[r, n]), (seed, r, n)


def test_each_group_uses_its_expert():
    """Expert e: all codes 8 except code 0 of column n, which is 8 + c_e, so
    W_e[0][n] = c_e * s and every other weight is 0; A[:, 0] = 2^(r mod 4),
    scales 2^-4: C[r][n] = 2^(r mod 4) * c_e / 16 exactly."""
    E, G, T, K, N, gs = 5, 7, 30, 64, 8, 32
    c_e = np.array([1, 2, 3, 5, 7])
    b = np.full((E, K // 8, N), 0x88888888, np.uint32)
    for e in range(E):
        b[e, 0, :] = 0x88888880 | (8 + c_e[e])
    s = np.full((E, K // gs, N), nm.f16_bits_of(np.array(2.0 ** -4)), np.uint16)
    a = np.zeros((T, K))
    a[:, 0] = 2.0 ** (np.arange(T) % 4)
    a_bits = nm.f16_bits_of(a)
    off = np.array([0, 3, 3, 9, 17, 20, 26, 30], np.uint32)
    ids = np.array([4, 0, -1, 2, 1, 3, 0], np.int32)
    c0 = np.full((T, N), SENT, np.uint16)
    got = oracle.grouped_gemm_w4(c0, a_bits, off, b, s, ids, np.array([8, G], np.uint32), gs)
    for g in range(G):
        for r in range(off[g], off[g + 1]):
            if ids[g] < 0:
                assert np.all(got[r] == SENT)
            else:
                want = 2.0 ** (r % 4) * c_e[ids[g]] / 16
                assert np.all(nm.decode_f16(got[r]) == want), (g, r)


def test_epilogue_each_group_uses_its_experts_bias_and_gate():
    """Zero activations: y = bias[e]; the gated output is silu(bias[e][2j]) * bias[e][2j+1]
    plus the residual, rounded once; skipped rows keep C."""
    import math
    a, off, b, s, ids, gs = _tiny(9)
    a[:] = 0
    T, N, E = a.shape[0], b.shape[2], b.shape[0]
    flags = oracle.EPI_BIAS | oracle.EPI_SILU_GATE | oracle.EPI_RESIDUAL
    bias, res = synth.grouped_epilogue_operands(2, E, T, N // 2, N, dtype="f16")
    c0 = np.full((T, N // 2), SENT, np.uint16)
    c = oracle.grouped_gemm_w4(c0, a, off, b, s, ids, np.array([T, len(ids)], np.uint32), gs, epilogue=flags,
                               bias_bits=bias, residual_bits=res)
    bf, rf = nm.decode_f16(bias), nm.decode_f16(res)
    for g, e in enumerate(ids):
        for r in range(off[g], off[g + 1]):
            if e < 0:
                assert np.all(c[r] == SENT)
                continue
            # silu(g) = g * sigmoid(g), sigmoid(g) = (1 + tanh(g / 2)) / 2
            x = [bf[e, 2 * j] * 0.5 * (1 + math.tanh(0.5 * bf[e, 2 * j])) * bf[e, 2 * j + 1] + rf[r, j]
                 for j in range(N // 2)]
            assert np.array_equal(c[r], nm.f16_bits_of(nm.round_to_f16(np.array(x)))), (g, r)


# ------------------------------------------------------------------ bf16 activations, scales and output

def test_bf16_single_group_reduces_to_w4():
    w = synth.w4_inputs(24, 40, 256, seed=12, group_size=64, dtype="bf16")
    T, N = w.a.shape[0], w.b.shape[1]
    got = oracle.grouped_gemm_w4(np.full((T, N), SENT, np.uint16), w.a, np.array([0, T], np.uint32),
                                 w.b[None], w.scales[None], np.array([0], np.int32), np.array([T, 1], np.uint32), 64,
                                 dtype="bf16")
    assert np.array_equal(got, oracle.qgemm_w4(w.a, w.b, w.scales, 64, dtype="bf16"))


def test_bf16_brute_force_tiny():
    """bf16 operands decoded by shifting the bits into a float32; scalar loops with
    their own nibble extraction. Every written value must be a nearest bf16 to
    the exact sum: no closer value is one bit pattern up or down."""
    for seed in range(3):
        rng = np.random.default_rng(100 + seed)
        E, G, T, K, N, gs = 3, 4, 18, 64, 8, 32
        counts = rng.multinomial(T, [1.0 / G] * G)
        off = np.zeros(G + 1, np.uint32)
        off[1:] = np.cumsum(counts)
        ids = rng.integers(-1, E, size=G).astype(np.int32)
        a = synth.bf16_bits(rng.standard_normal((T, K)))
        b = rng.integers(0, 2**32, size=(E, K // 8, N), dtype=np.uint32)
        s = synth.bf16_bits(rng.uniform(0.005, 0.02, size=(E, K // gs, N)))
        c0 = np.full((T, N), SENT, np.uint16)
        got = oracle.grouped_gemm_w4(c0, a, off, b, s, ids, np.array([0, G], np.uint32), gs, dtype="bf16")
        av = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        sv = (s.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        dec = lambda v: float((np.uint32(v) << 16).view(np.float32))
        written = np.zeros((T, N), bool)
        for g in range(G):
            e = int(ids[g])
            if e < 0:
                continue
            for r in range(int(off[g]), int(off[g + 1])):
                written[r] = True
                for n in range(N):
                    acc = 0.0
                    for k in range(K):
                        q = (int(b[e, k // 8, n]) >> (4 * (k % 8))) & 0xF
                        acc += av[r, k] * (q - 8) * sv[e, k // gs, n]
                    v = int(got[r, n])
                    err = abs(acc - dec(v))
                    for nb in (v - 1, v + 1):
                        if 0 <= nb < 0x10000 and (nb & 0x7FFF) < 0x7F80:   # finite neighbours
                            assert err <= abs(acc - dec(nb)), (seed, r, n)
        assert np.all(got[~written] == SENT)


def test_bf16_each_group_uses_its_expert_exactly():
    """The expert fingerprint of the fp16 pin above in bf16: C[r][n] = 2^(r mod 4) c_e / 16, exact."""
    E, G, T, K, N, gs = 5, 7, 30, 64, 8, 32
    c_e = np.array([1, 2, 3, 5, 7])
    b = np.full((E, K // 8, N), 0x88888888, np.uint32)
    for e in range(E):
        b[e, 0, :] = 0x88888880 | (8 + c_e[e])
    s = np.full((E, K // gs, N), nm.bf16_bits_of(np.array(2.0 ** -4)), np.uint16)
    a = np.zeros((T, K))
    a[:, 0] = 2.0 ** (np.arange(T) % 4)
    off = np.array([0, 3, 3, 9, 17, 20, 26, 30], np.uint32)
    ids = np.array([4, 0, -1, 2, 1, 3, 0], np.int32)
    c0 = np.full((T, N), SENT, np.uint16)
    got = oracle.grouped_gemm_w4(c0, nm.bf16_bits_of(a), off, b, s, ids, np.array([8, G], np.uint32), gs,
                                 dtype="bf16")
    for g in range(G):
        for r in range(off[g], off[g + 1]):
            if ids[g] < 0:
                assert np.all(got[r] == SENT)
            else:
                assert np.all(nm.decode_bf16(got[r]) == 2.0 ** (r % 4) * c_e[ids[g]] / 16), (g, r)
