"""Plant plausible mistakes in the oracle (on the CPU) and check that at least one
pin fails for each: evidence that the pins constrain the oracle."""
import numpy as np
import pytest

import oracle
from oracle import numerics as nm
from oracle import w4 as ow4
from oracle import kproj as okp
import test_oracle_w4 as tw4
import test_oracle_kproj as tkp
import test_oracle_numerics as tnm

_orig_dequant = ow4.dequant_w4


def _dequant_variant(kind):
    def f(b_packed, scales_bits, group_size, pack_factor=8, dtype="f16"):
        b = np.asarray(b_packed, dtype=np.uint32)
        K = b.shape[0] * 8
        s = nm.decode_bf16(scales_bits) if dtype == "bf16" and kind != "bf16_as_f16" else nm.decode_f16(scales_bits)
        order = np.arange(8)[::-1] if kind == "nibble_order" else np.arange(8)
        shifts = (4 * order.astype(np.uint32))[None, :, None]
        q = ((b[:, None, :] >> shifts) & np.uint32(0xF)).astype(np.int64).reshape(K, -1)
        zp = 7 if kind == "zero_point" else 8
        gsz = group_size // 2 if kind == "group_index" else group_size
        gidx = np.minimum(np.arange(K) // gsz, s.shape[0] - 1)
        w = (q - zp).astype(np.float64) * s[gidx, :]
        if kind == "signed_code":
            w = np.where(q >= 8, q - 16, q).astype(np.float64) * s[gidx, :]
        return w
    return f


W4_PINS = [tw4.test_worked_examples_from_fixture, tw4.test_nibble_position,
           tw4.test_identity_gives_unpacked_weights_exactly, tw4.test_closed_form_ones_and_power_of_two_scales]


W4_BF16_PINS = [lambda: tw4.test_bf16_brute_force_small(3, 5, 256, 64), tw4.test_bf16_unit_rows_read_codes_back]


@pytest.mark.parametrize("kind", ["nibble_order", "zero_point", "group_index", "signed_code", "bf16_as_f16"])
def test_w4_mutation_is_caught(kind, monkeypatch):
    monkeypatch.setattr(ow4, "dequant_w4", _dequant_variant(kind))
    failures = 0
    for pin in (W4_BF16_PINS if kind == "bf16_as_f16" else W4_PINS):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1, kind


def _epilogue_variant(kind):
    def f(a_bits, b_packed, scales_bits, group_size, epilogue, bias_bits=None, residual_bits=None,
          pack_factor=8, dtype="f16"):
        dec = ow4._DECODE[dtype]
        rnd, bits_of = ow4._ROUND[dtype]
        y = ow4.qgemm_w4_f64(a_bits, b_packed, scales_bits, group_size, pack_factor, dtype)
        if kind == "early_rounding":
            y = rnd(y)
        silu = (lambda x: x / (1.0 + np.exp(x))) if kind == "silu_sign" else ow4.silu
        if epilogue & ow4.EPI_BIAS and kind != "bias_after_gate":
            y = y + dec(bias_bits)[None, :]
        if epilogue & ow4.EPI_SILU_GATE:
            z = silu(y[:, 1::2]) * y[:, 0::2] if kind == "gate_swapped" else silu(y[:, 0::2]) * y[:, 1::2]
        else:
            z = y
        if epilogue & ow4.EPI_BIAS and kind == "bias_after_gate":
            z = z + dec(bias_bits)[None, :z.shape[1]]
        if epilogue & ow4.EPI_RESIDUAL:
            z = z + dec(residual_bits)
        return bits_of(rnd(z))
    return f


EPI_PINS = [lambda: [tw4.test_epilogue_brute_force_every_flag_set(f) for f in range(8)],
            tw4.test_epilogue_zero_activations_give_bias_and_residual, tw4.test_epilogue_gate_pairs_gate_then_up,
            tw4.test_epilogue_bias_is_added_before_the_gate]


@pytest.mark.parametrize("kind", ["gate_swapped", "bias_after_gate", "silu_sign", "early_rounding"])
def test_epilogue_mutation_is_caught(kind, monkeypatch):
    monkeypatch.setattr(oracle, "qgemm_w4_epilogue", _epilogue_variant(kind))
    failures = 0
    for pin in EPI_PINS:
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1, kind


def test_round_mutation_is_caught(monkeypatch):
    """Round half away from zero instead of half to even."""
    def bad(x, fmt):
        x = np.asarray(x, dtype=np.float64)
        _, e = np.frexp(x)
        q = np.ldexp(1.0, np.maximum(e - 1, fmt.emin) - (fmt.p - 1))
        return np.sign(x) * np.floor(np.abs(x) / q + 0.5) * q
    monkeypatch.setattr(nm, "round_to", bad)
    with pytest.raises(AssertionError):
        tnm.test_round_f16_brute_force_and_numpy()


def test_kproj_mutations_are_caught(monkeypatch):
    # page index taken from the token index instead of the cache position
    orig = okp.token_slots

    def bad_slots(row_offsets, cache_lengths, page_table, page_size):
        return orig(row_offsets, np.zeros_like(np.asarray(cache_lengths)), page_table, page_size)
    monkeypatch.setattr(okp, "token_slots", bad_slots)
    with pytest.raises(AssertionError):
        tkp.test_placement_fingerprint_and_untouched_bytes()
    monkeypatch.setattr(okp, "token_slots", orig)

    # weight scale indexed with a transposed block index
    orig_exact = okp.kproj_exact

    def bad_exact(hidden_bits, weight_codes, input_scale, weight_scale, granularity=(1, 128, 128)):
        return orig_exact(hidden_bits, weight_codes, input_scale, np.ascontiguousarray(weight_scale.T), granularity)
    monkeypatch.setattr(okp, "kproj_exact", bad_exact)
    with pytest.raises(AssertionError):
        tkp.test_brute_force_loops()


def _quantize_variant(kind):
    def f(values, G):
        x32 = np.asarray(values, dtype=np.float64).astype(np.float32)
        T, n = x32.shape
        runs = x32.reshape(T, G, n // G).transpose(0, 2, 1) if kind == "run_stride" else x32.reshape(T, n // G, G)
        amax = np.abs(runs).max(axis=2)
        s = (amax / np.float32(240.0 if kind == "fnuz_max" else 448.0)).astype(np.float32)
        safe = np.where(s > 0, s, np.float32(1.0))
        v = np.where(s[:, :, None] > 0, runs / safe[:, :, None], np.float32(0.0)).astype(np.float64)
        codes = nm.encode_e4m3(v)
        if kind == "truncate":   # round toward zero: step back every code that rounded up in magnitude
            over = (np.abs(nm.decode_e4m3(codes)) > np.abs(v)) & ((codes & 0x7F) > 0)
            codes = np.where(over, codes - 1, codes).astype(np.uint8)
        if kind == "run_stride":
            codes = codes.reshape(T, n // G, G).transpose(0, 2, 1)
        return codes.reshape(T, n), s
    return f


E4M3_CACHE_PINS = [tkp.test_e4m3_cache_reproduces_exact_codes, tkp.test_e4m3_cache_rounds_to_nearest_even_and_zero_runs]


@pytest.mark.parametrize("kind", ["fnuz_max", "truncate", "run_stride"])
def test_e4m3_cache_mutation_is_caught(kind, monkeypatch):
    monkeypatch.setattr(okp, "quantize_runs", _quantize_variant(kind))
    failures = 0
    for pin in E4M3_CACHE_PINS:
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1, kind


def test_kv_plane_swap_is_caught(monkeypatch):
    orig_exact = okp.kproj_exact

    def swapped(hidden_bits, weight_codes, input_scale, weight_scale, granularity=(1, 128, 128)):
        x = orig_exact(hidden_bits, weight_codes, input_scale, weight_scale, granularity)
        h = x.shape[1] // 2
        return np.concatenate([x[:, h:], x[:, :h]], axis=1)
    monkeypatch.setattr(okp, "kproj_exact", swapped)
    with pytest.raises(AssertionError):
        tkp.test_kv_planes_fingerprint_and_untouched_bytes()


def _grouped_w4_variant(kind):
    from oracle import grouped_w4 as og
    orig = og.grouped_gemm_w4

    def f(c_bits, a_bits, a_offsets, b_packed, scales_bits, expert_ids, usage_stats, group_size):
        ids = np.array(expert_ids, dtype=np.int32, copy=True)
        if kind == "expert_is_group":
            ids = np.where(ids >= 0, np.arange(len(ids)) % np.asarray(b_packed).shape[0], ids).astype(np.int32)
        elif kind == "no_skip":
            ids = np.where(ids < 0, 0, ids).astype(np.int32)
        return orig(c_bits, a_bits, a_offsets, b_packed, scales_bits, ids, usage_stats, group_size)
    return f


@pytest.mark.parametrize("kind", ["expert_is_group", "no_skip"])
def test_grouped_w4_mutation_is_caught(kind, monkeypatch):
    import test_oracle_grouped_w4 as tgw
    monkeypatch.setattr(oracle, "grouped_gemm_w4", _grouped_w4_variant(kind))
    failures = 0
    for pin in (tgw.test_skip_semantics, tgw.test_each_group_uses_its_expert):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1, kind


def _plane_columns_variant(kind):
    from oracle import grouped as og
    orig = og.plane_columns

    def f(a_plane_splits, n):
        r = orig(a_plane_splits, n)
        if len(r) == 1:
            return r
        (a0, a1), (b0, b1), (c0, c1) = r
        if kind == "boundary_off_by_one":
            return [(a0, a1 + 1), (b0 + 1, b1), (c0, c1)] if a1 < b1 else r
        if kind == "planes_reversed":      # the first column range reads plane 2, the last plane 0
            return [(c0, c1), (b0, b1), (a0, a1)]
        if kind == "second_split_absolute":  # s1 taken as an end column instead of a size
            s1 = b1 - b0
            return [(a0, a1), (a1, max(a1, s1)), (max(a1, s1), n)]
        return r
    return f


@pytest.mark.parametrize("kind", ["boundary_off_by_one", "planes_reversed", "second_split_absolute"])
def test_plane_split_mutation_is_caught(kind, monkeypatch):
    import test_oracle_grouped as tg
    from oracle import grouped as og
    monkeypatch.setattr(og, "plane_columns", _plane_columns_variant(kind))
    failed = 0
    for pin in (tg.test_planes_worked_example_from_fixture, tg.test_planes_route_columns_exactly,
                tg.test_planes_brute_force_integers):
        try:
            pin()
        except (AssertionError, ValueError):
            failed += 1
    assert failed > 0, f"no pin catches the {kind} mutation"
