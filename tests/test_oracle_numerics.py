"""Pins for the oracle's number formats: decoders against the libraries' own
decoders over every bit pattern, rounding against a brute-force nearest-value
search over every finite value of the format."""
import numpy as np
import pytest
import torch

from oracle import numerics as nm

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_decode_f16_all_patterns_match_numpy():
    ours = nm.decode_f16(ALL16)
    ref = ALL16.view(np.float16).astype(np.float64)
    assert np.array_equal(ours, ref, equal_nan=True)


def test_decode_bf16_all_patterns_match_torch():
    ours = nm.decode_bf16(ALL16)
    ref = torch.from_numpy(ALL16.view(np.int16).copy()).view(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(ours, ref, equal_nan=True)


def test_decode_e4m3_all_codes_match_torch_and_fixed_points():
    codes = np.arange(256, dtype=np.uint8)
    ours = nm.decode_e4m3(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(ours, ref, equal_nan=True)
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert np.sum(np.isnan(ours)) == 2
    # values fixed by the OCP E4M3 definition
    assert ours[0x38] == 1.0 and ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6 and ours[0x80] == 0.0


def _nearest_even(x, table_vals, table_bits, max_finite, half_ulp_max):
    """Brute force: nearest finite value, ties to the even bit pattern, overflow to inf."""
    out = np.empty_like(x)
    for i, v in enumerate(x):
        a = abs(v)
        if a >= max_finite + half_ulp_max:
            out[i] = np.copysign(np.inf, v)
            continue
        d = np.abs(table_vals - a)
        best = d.min()
        cand = np.nonzero(d == best)[0]
        if len(cand) > 1:
            cand = [c for c in cand if table_bits[c] % 2 == 0]
        out[i] = np.copysign(table_vals[cand[0]], v)
    return out


def _sample(rng, lo_exp, hi_exp, n):
    mag = np.ldexp(rng.uniform(1.0, 2.0, n), rng.integers(lo_exp, hi_exp, n))
    return mag * rng.choice([-1.0, 1.0], n)


def test_round_f16_brute_force_and_numpy():
    rng = np.random.default_rng(0)
    pos = ALL16[:0x7C00]                    # finite non-negative patterns
    vals = pos.view(np.float16).astype(np.float64)
    x = _sample(rng, -27, 17, 1500)
    # exact midpoints between neighbours (ties), incl. subnormal range and the top binade
    mids = (vals[1:] + vals[:-1]) / 2
    x = np.concatenate([x, rng.choice(mids, 500), -rng.choice(mids, 200), [65519.9, 65520.0, 2.0**-25, 3 * 2.0**-26]])
    bf = _nearest_even(x, vals, pos, 65504.0, 16.0)
    ours = nm.round_to_f16(x)
    assert np.array_equal(ours, bf)
    assert np.array_equal(ours, x.astype(np.float16).astype(np.float64))


def test_round_bf16_brute_force_and_torch():
    rng = np.random.default_rng(1)
    pos = ALL16[:0x7F80]
    vals = nm.decode_bf16(pos)
    x = _sample(rng, -135, 127, 1200)
    mids = (vals[1:] + vals[:-1]) / 2
    x = np.concatenate([x, rng.choice(mids, 400), -rng.choice(mids, 100)])
    bf = _nearest_even(x, vals, pos, float(vals[-1]), float(vals[-1] - vals[-2]) / 2)
    ours = nm.round_to_bf16(x)
    assert np.array_equal(ours, bf)
    # torch's float32 -> bfloat16 cast is also nearest-even; compare on float32-exact inputs
    x32 = x.astype(np.float32)
    x32 = x32[np.isfinite(x32)]
    tb = torch.from_numpy(x32).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(nm.round_to_bf16(x32.astype(np.float64)), tb)


def test_round_keeps_signed_zero_and_representable_values():
    assert np.signbit(nm.round_to_f16(np.array([-0.0]))[0])
    assert np.signbit(nm.round_to_f16(np.array([-1e-30]))[0])
    vals = ALL16[:0x7C00].view(np.float16).astype(np.float64)
    assert np.array_equal(nm.round_to_f16(vals), vals)


def test_bits_of_roundtrip():
    vals = ALL16[:0x7C00].view(np.float16).astype(np.float64)
    assert np.array_equal(nm.f16_bits_of(vals), ALL16[:0x7C00])
    bvals = nm.decode_bf16(ALL16[:0x7F80])
    assert np.array_equal(nm.bf16_bits_of(bvals), ALL16[:0x7F80])
    with pytest.raises(AssertionError):
        nm.f16_bits_of(np.array([1.0 + 2.0 ** -12]))


def test_encode_e4m3_matches_torch_and_ties_to_even():
    """Every finite code round-trips; a dense sweep of values (and every midpoint
    between neighbouring codes) rounds as torch's float8_e4m3fn cast does."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(nm.encode_e4m3(nm.decode_e4m3(codes)), codes)
    pos = np.sort(nm.decode_e4m3(np.arange(0, 0x7F, dtype=np.uint8)))       # 0 .. 448
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(0)
    sweep = np.concatenate([mids, -mids, rng.uniform(-448, 448, 20000), rng.uniform(-0.05, 0.05, 20000),
                            [448.0, -448.0, 0.0, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -6 * 0.999]])
    ref = torch.from_numpy(sweep.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = nm.encode_e4m3(sweep.astype(np.float32).astype(np.float64))
    assert np.array_equal(got, ref)
    # ties to the even code: 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39)
    assert nm.encode_e4m3(np.array([1.0625, 1.1875, -1.0625]))[:].tolist() == [0x38, 0x3A, 0xB8]
    # saturation just above the largest finite value, signed zero kept
    assert nm.encode_e4m3(np.array([448.0 * (1 + 2.0 ** -20), -1e-9, 0.0])).tolist() == [0x7E, 0x80, 0x00]
