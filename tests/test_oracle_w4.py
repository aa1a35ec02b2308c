"""Pins for the W4A16 oracle (Modular page "multistage_gemm_q": group_size and
pack_factor parameters; rank-2 requirement in its Raises section).

Each pin is chosen so that a plausible slip in the oracle (nibble order, the
zero point, the group index, a transposed operand, a dropped group) fails."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import numerics as nm
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "w4_worked_examples.json")
ONE = 0x3C00  # fp16 1.0


def _const(shape, v, dtype):
    return np.full(shape, v, dtype=dtype)


def _brute(a_bits, b, s_bits, gs):
    """Scalar loops; codes read as hexadecimal digits counted from the right."""
    M, K = a_bits.shape
    N = b.shape[1]
    a = a_bits.view(np.float16).astype(np.float64)
    s = s_bits.view(np.float16).astype(np.float64)
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                digits = "%08x" % int(b[k // 8, n])
                q = int(digits[7 - (k % 8)], 16)
                acc += float(a[m, k]) * (q - 8) * float(s[k // gs, n])
            out[m, n] = acc
    return out


def test_worked_examples_from_fixture():
    ex = json.load(open(GOLD))["examples"]
    assert len(ex) >= 4
    for e in ex:
        K, N, M, gs = e["K"], e["N"], e["M"], e["group_size"]
        b = _const((K // 8, N), int(e["word"], 16), np.uint32)
        if "scale_bits_per_group" in e:
            s = np.array([[int(v, 16)] * N for v in e["scale_bits_per_group"]], dtype=np.uint16)
        else:
            s = _const((K // gs, N), int(e["scale_bits"], 16), np.uint16)
        a = _const((M, K), int(e["a_bits"], 16), np.uint16)
        c = oracle.qgemm_w4(a, b, s, gs)
        assert [hex(v) for v in c.ravel()] == [hex(int(v, 16)) for v in e["expected_bits"]], e["name"]


@pytest.mark.parametrize("M,N,K,gs", [(1, 3, 128, 128), (3, 5, 256, 128), (2, 4, 256, 64), (4, 2, 64, 32)])
def test_brute_force_small(M, N, K, gs):
    w = synth.w4_inputs(M, N, K, seed=11 + M, group_size=gs)
    got = oracle.w4.qgemm_w4_f64(w.a, w.b, w.scales, gs)
    ref = _brute(w.a, w.b, w.scales, gs)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(oracle.qgemm_w4(w.a, w.b, w.scales, gs), nm.f16_bits_of(nm.round_to_f16(ref)))


def test_nibble_position():
    """Only code j of each word is 9 (weight +1 * scale); a unit A row picks out one K row."""
    K, gs = 128, 128
    for j in range(8):
        b = _const((K // 8, 1), 0x88888888 + (1 << (4 * j)), np.uint32)
        s = _const((1, 1), ONE, np.uint16)
        a = np.zeros((8, K), dtype=np.uint16)
        for jj in range(8):
            a[jj, 8 * 5 + jj] = ONE          # rows of word kp = 5
        c = oracle.qgemm_w4(a, b, s, gs).view(np.float16).astype(np.float64).ravel()
        expect = np.zeros(8)
        expect[j] = 1.0
        assert np.array_equal(c, expect), j


def test_identity_gives_unpacked_weights_exactly():
    """A = I_K: C[k, n] = round_fp16((q - 8) * scale) for every k, n."""
    K, N, gs = 256, 8, 128
    w = synth.w4_inputs(1, N, K, seed=3, group_size=gs)
    a = np.zeros((K, K), dtype=np.uint16)
    np.fill_diagonal(a, ONE)
    c = oracle.qgemm_w4(a, w.b, w.scales, gs).view(np.float16).astype(np.float64)
    s = w.scales.view(np.float16).astype(np.float64)
    for k in range(K):
        for n in range(N):
            q = (int(w.b[k // 8, n]) >> (4 * (k % 8))) & 15
            assert c[k, n] == np.float64(np.float16((q - 8) * s[k // gs, n]))


def test_zero_scale_equals_zero_activation_block():
    M, N, K, gs = 4, 16, 512, 128
    w = synth.w4_inputs(M, N, K, seed=5, group_size=gs)
    for g in range(K // gs):
        s0 = w.scales.copy()
        s0[g] = 0
        a0 = w.a.copy()
        a0[:, g * gs:(g + 1) * gs] = 0
        c1 = oracle.w4.qgemm_w4_f64(w.a, w.b, s0, gs)
        c2 = oracle.w4.qgemm_w4_f64(a0, w.b, w.scales, gs)
        assert np.allclose(c1, c2, rtol=1e-13, atol=1e-13)
        # and the removed part is that group's own product
        full = oracle.w4.qgemm_w4_f64(w.a, w.b, w.scales, gs)
        a_only = np.zeros_like(w.a)
        a_only[:, g * gs:(g + 1) * gs] = w.a[:, g * gs:(g + 1) * gs]
        part = oracle.w4.qgemm_w4_f64(a_only, w.b, w.scales, gs)
        assert np.allclose(full - part, c1, rtol=1e-12, atol=1e-12)


def test_scale_linearity_is_exact():
    M, N, K, gs = 3, 8, 256, 128
    w = synth.w4_inputs(M, N, K, seed=6, group_size=gs)
    s2 = nm.f16_bits_of(2 * w.scales.view(np.float16).astype(np.float64))
    c1 = oracle.qgemm_w4(w.a, w.b, w.scales, gs).view(np.float16).astype(np.float64)
    c2 = oracle.qgemm_w4(w.a, w.b, s2, gs).view(np.float16).astype(np.float64)
    assert np.array_equal(c2, 2 * c1)


def test_closed_form_ones_and_power_of_two_scales():
    """A = ones and scales = distinct powers of two: C[n] = sum_g s[g][n] * sum_{k in g} (q - 8)."""
    N, K, gs = 6, 512, 128
    rng = np.random.default_rng(7)
    b = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
    G = K // gs
    exps = rng.integers(-8, -2, size=(G, N))
    s = nm.f16_bits_of(np.ldexp(1.0, exps))
    a = _const((1, K), ONE, np.uint16)
    c64 = oracle.w4.qgemm_w4_f64(a, b, s, gs)[0]
    c = oracle.qgemm_w4(a, b, s, gs).view(np.float16).astype(np.float64)[0]
    for n in range(N):
        total = 0.0
        for g in range(G):
            qsum = 0
            for kp in range(g * gs // 8, (g + 1) * gs // 8):
                word = int(b[kp, n])
                qsum += sum(((word >> (4 * i)) & 15) - 8 for i in range(8))
            total += qsum * 2.0 ** int(exps[g, n])
        assert c64[n] == total                       # exact: dyadic terms
        assert c[n] == np.float64(np.float16(total))  # one nearest-even rounding


def test_column_permutation():
    M, N, K, gs = 2, 12, 256, 128
    w = synth.w4_inputs(M, N, K, seed=8, group_size=gs)
    perm = np.random.default_rng(0).permutation(N)
    c = oracle.qgemm_w4(w.a, w.b, w.scales, gs)
    cp = oracle.qgemm_w4(w.a, w.b[:, perm], w.scales[:, perm], gs)
    assert np.array_equal(cp, c[:, perm])


def test_rank2_is_required():
    w = synth.w4_inputs(2, 8, 128, seed=1)
    with pytest.raises(ValueError):
        oracle.qgemm_w4(w.a[None], w.b, w.scales, 128)
    with pytest.raises(ValueError):
        oracle.qgemm_w4(w.a, w.b.ravel(), w.scales, 128)


# ---- bf16 activations / scales / result (the page's a_type and c_type) ----

def _bf16_to_f64(bits):
    """bfloat16 bit patterns -> float64 by placing them in the top half of a float32."""
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("M,N,K,gs", [(1, 3, 128, 128), (3, 5, 256, 64), (2, 4, 64, 32)])
def test_bf16_brute_force_small(M, N, K, gs):
    """Scalar loops over the bf16 inputs (decoded here by bit placement, not by
    the oracle's decoder) against the oracle's unrounded product."""
    w = synth.w4_inputs(M, N, K, seed=31 + M, group_size=gs, dtype="bf16")
    a = _bf16_to_f64(w.a)
    s = _bf16_to_f64(w.scales)
    ref = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                q = (int(w.b[k // 8, n]) >> (4 * (k % 8))) & 0xF
                acc += a[m, k] * (q - 8) * s[k // gs, n]
            ref[m, n] = acc
    got = oracle.w4.qgemm_w4_f64(w.a, w.b, w.scales, gs, dtype="bf16")
    assert np.allclose(got, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))


def test_bf16_unit_rows_read_codes_back():
    """A = identity rows: row k of C is W[k, :] = (q - 8) * s, which is exact in
    bf16 whenever s is a power of two."""
    K, N, gs = 64, 16, 32
    rng = np.random.default_rng(5)
    b = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
    s_vals = 2.0 ** rng.integers(-6, 0, size=(K // gs, N))
    s = synth.bf16_bits(s_vals)
    a = synth.bf16_bits(np.eye(K))
    c = _bf16_to_f64(oracle.qgemm_w4(a, b, s, gs, dtype="bf16"))
    codes = np.array([[(int(b[k // 8, n]) >> (4 * (k % 8))) & 0xF for n in range(N)] for k in range(K)])
    assert np.array_equal(c, (codes - 8) * s_vals[np.arange(K) // gs])


def test_bf16_result_rounding_differs_from_f16():
    """The same exactly representable inputs give the bf16-rounded product: a sum
    whose exact value needs more than 8 significant bits rounds to nearest even."""
    K, N, gs = 32, 1, 32
    # one active code per row: a = [1 + 2^-7] at k = 0, code 9 (weight +1 * s), s = 1
    a = np.zeros((1, K))
    a[0, 0] = 1.0 + 2.0 ** -7
    a[0, 1] = 2.0 ** -9          # tips the sum to 1 + 2^-7 + 2^-9: between bf16 neighbours
    b = np.full((K // 8, N), 0x88888888, np.uint32)   # code 8 (weight 0) everywhere...
    b[0, 0] = 0x88888899                               # ...but codes 9 at k = 0 and k = 1
    s = synth.bf16_bits(np.ones((1, N)))
    got = _bf16_to_f64(oracle.qgemm_w4(synth.bf16_bits(a), b, s, gs, dtype="bf16"))[0, 0]
    exact = 1.0 + 2.0 ** -7 + 2.0 ** -9
    assert got == 1.0 + 2.0 ** -7             # bf16 nearest of the exact sum (8 significant bits)
    f16 = oracle.qgemm_w4(synth.f16_bits(a), b, synth.f16_bits(np.ones((1, N))), gs).view(np.float16)[0, 0]
    assert float(f16) == exact                # fp16 keeps it


# ---------------------------------------------------------------- fixed epilogues
# The page's optional per-element epilogue is offered as three fixed steps
# (bias, SiLU-gated column pairs, residual); these pins check the oracle's
# version against independent scalar code and closed forms.

def _sigmoid_tanh(x):
    """sigmoid(x) = (1 + tanh(x / 2)) / 2: a second, independent formula."""
    import math
    return 0.5 * (1.0 + math.tanh(0.5 * x))


def test_silu_closed_forms():
    import math
    xs = np.array([-30.0, -3.0, -1.0, -0.25, 0.0, 0.5, 1.0, 2.0, 7.5, 40.0])
    got = oracle.silu(xs)
    for x, g in zip(xs, got):
        assert abs(g - x * _sigmoid_tanh(x)) <= 1e-15 * (1 + abs(x))
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    # silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1)
    assert np.allclose(oracle.silu(xs) - oracle.silu(-xs), xs, rtol=0, atol=1e-13)


def _brute_epilogue(a_bits, b, s_bits, gs, flags, bias_bits, res_bits):
    y = _brute(a_bits, b, s_bits, gs)
    M, N = y.shape
    if flags & oracle.EPI_BIAS:
        bias = bias_bits.view(np.float16).astype(np.float64)
        for n in range(N):
            y[:, n] += bias[n]
    if flags & oracle.EPI_SILU_GATE:
        z = np.zeros((M, N // 2))
        for m in range(M):
            for j in range(N // 2):
                g, u = y[m, 2 * j], y[m, 2 * j + 1]
                z[m, j] = g * _sigmoid_tanh(g) * u
    else:
        z = y
    if flags & oracle.EPI_RESIDUAL:
        z = z + res_bits.view(np.float16).astype(np.float64)
    return z


@pytest.mark.parametrize("flags", range(8))
def test_epilogue_brute_force_every_flag_set(flags):
    M, N, K, gs = 3, 8, 128, 64
    w = synth.w4_inputs(M, N, K, seed=40 + flags, group_size=gs)
    n_out = N // 2 if flags & oracle.EPI_SILU_GATE else N
    bias, res = synth.w4_epilogue_operands(50 + flags, M, n_out, N)
    got = oracle.qgemm_w4_epilogue(w.a, w.b, w.scales, gs, flags, bias, res)
    exact = _brute_epilogue(w.a, w.b, w.scales, gs, flags, bias, res)
    assert got.shape == (M, n_out)
    # one rounding of the exact value: within half an fp16 ulp of it
    diff = np.abs(got.view(np.float16).astype(np.float64) - exact)
    ulp = np.spacing(np.abs(exact).astype(np.float16)).astype(np.float64)
    assert np.all(diff <= 0.5 * ulp + 1e-12), flags
    if flags == 0:
        assert np.array_equal(got, oracle.qgemm_w4(w.a, w.b, w.scales, gs))


def test_epilogue_zero_activations_give_bias_and_residual():
    M, N, K, gs = 2, 16, 128, 128
    w = synth.w4_inputs(M, N, K, seed=3, group_size=gs)
    w.a[:] = 0
    bias, res = synth.w4_epilogue_operands(7, M, N, N)
    assert np.array_equal(oracle.qgemm_w4_epilogue(w.a, w.b, w.scales, gs, oracle.EPI_BIAS, bias, None),
                          np.broadcast_to(bias, (M, N)))
    assert np.array_equal(oracle.qgemm_w4_epilogue(w.a, w.b, w.scales, gs, oracle.EPI_RESIDUAL, None, res), res)
    # Y = 0: the gate gives silu(0) * 0 = 0, then the residual
    bias2, res2 = synth.w4_epilogue_operands(8, M, N // 2, N)
    got = oracle.qgemm_w4_epilogue(w.a, w.b, w.scales, gs, oracle.EPI_SILU_GATE | oracle.EPI_RESIDUAL, None, res2)
    assert np.array_equal(got, res2)


def test_epilogue_gate_pairs_gate_then_up():
    """A unit row picks one K row of weights, so Y[2j] and Y[2j+1] are known codes:
    the gate must take silu of the even column and scale it by the odd one."""
    K, N, gs = 128, 16, 128
    w = synth.w4_inputs(1, N, K, seed=5, group_size=gs)
    w.a = np.zeros((1, K), np.uint16)
    w.a[0, 0] = ONE
    w.b[0, 0::2] = (w.b[0, 0::2] & ~np.uint32(0xF)) | np.uint32(0xF)   # k = 0 code 15: gate 7
    w.b[0, 1::2] = (w.b[0, 1::2] & ~np.uint32(0xF)) | np.uint32(0xB)   # k = 0 code 11: up 3
    w.scales[:] = ONE
    y = oracle.w4.qgemm_w4_f64(w.a, w.b, w.scales, gs)
    assert np.all(y[0, 0::2] == 7.0) and np.all(y[0, 1::2] == 3.0)
    got = oracle.qgemm_w4_epilogue(w.a, w.b, w.scales, gs, oracle.EPI_SILU_GATE).view(np.float16)
    g, u = 7.0, 3.0
    assert np.all(got == np.float16(g * _sigmoid_tanh(g) * u))
    assert np.float16(g * _sigmoid_tanh(g) * u) != np.float16(u * _sigmoid_tanh(u) * g)


def test_epilogue_bias_is_added_before_the_gate():
    M, N, K, gs = 1, 16, 128, 128
    w = synth.w4_inputs(M, N, K, seed=6, group_size=gs)
    w.a[:] = 0
    bias = np.array([0x4000, 0x4200] * (N // 2), np.uint16)   # gate 2, up 3
    got = oracle.qgemm_w4_epilogue(w.a, w.b, w.scales, gs, oracle.EPI_BIAS | oracle.EPI_SILU_GATE, bias, None)
    assert np.all(got.view(np.float16) == np.float16(2.0 * _sigmoid_tanh(2.0) * 3.0))


# ---------------------------------------------------------------- [N, K/8] storage

def test_nk_layout_brute_force():
    """Scalar loops reading word (n, k // 8) of the [N, K/8] array and scale (n, k // gs)."""
    for (M, N, K, gs) in [(2, 5, 64, 32), (3, 8, 128, 64)]:
        w = synth.w4_inputs(M, N, K, seed=M + N, group_size=gs)
        b_nk = np.ascontiguousarray(w.b.T)
        s_nk = np.ascontiguousarray(w.scales.T)
        a = w.a.view(np.float16).astype(np.float64)
        s = s_nk.view(np.float16).astype(np.float64)
        ref = np.zeros((M, N))
        for m in range(M):
            for n in range(N):
                for k in range(K):
                    q = (int(b_nk[n, k // 8]) >> (4 * (k % 8))) & 0xF
                    ref[m, n] += a[m, k] * (q - 8) * s[n, k // gs]
        got = oracle.qgemm_w4_nk(w.a, b_nk, s_nk, gs).view(np.float16).astype(np.float64)
        assert np.array_equal(got, nm.round_to_f16(ref))
