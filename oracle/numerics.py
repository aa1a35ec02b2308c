"""Number formats used by the three operations, written from their definitions.

* IEEE 754 binary16 (fp16): 1 sign, 5 exponent (bias 15), 10 fraction bits.
* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits.
* OCP FP8 E4M3 ("fn" variant): 1 sign, 4 exponent (bias 7), 3 fraction bits,
  no infinities, S.1111.111 is NaN, max finite 448.

Rounding to an output format is round-to-nearest, ties-to-even, done directly
from float64 (never through float32, which could round twice). None of the
pages states an output rounding; nearest-even is the IEEE default and is the
reading used throughout.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Fmt:
    name: str
    p: int          # significand precision in bits (including the implicit bit)
    emin: int       # exponent of the smallest normal number
    max_finite: float


F16 = Fmt("f16", p=11, emin=-14, max_finite=65504.0)
BF16 = Fmt("bf16", p=8, emin=-126, max_finite=float(np.ldexp(255.0, 120)))  # (2 - 2^-7) * 2^127
E4M3 = Fmt("e4m3", p=4, emin=-6, max_finite=448.0)


def round_to(x, fmt: Fmt) -> np.ndarray:
    """Round float64 values to the nearest value of `fmt` (ties to even); returns float64.

    With x = m * 2^e (0.5 <= |m| < 1), the spacing of `fmt` around x is
    2^(max(e-1, emin) - (p-1)); dividing by that power of two, rounding to the
    nearest integer (numpy rint is ties-to-even) and multiplying back are all
    exact in float64. Results above the largest finite value become +-inf,
    as IEEE nearest rounding does. Zero keeps its sign.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    E = np.maximum(e - 1, fmt.emin)
    quantum = np.ldexp(1.0, E - (fmt.p - 1))
    r = np.rint(x / quantum) * quantum
    r = np.where(np.abs(r) > fmt.max_finite, np.copysign(np.inf, x), r)
    r = np.where(x == 0, x, r)
    return r


def round_to_f16(x) -> np.ndarray:
    return round_to(x, F16)


def round_to_bf16(x) -> np.ndarray:
    return round_to(x, BF16)


def f16_bits_of(r: np.ndarray) -> np.ndarray:
    """Bit patterns of float64 values that are already exactly representable in fp16."""
    r = np.asarray(r, dtype=np.float64)
    h = r.astype(np.float16)
    assert np.array_equal(h.astype(np.float64), r, equal_nan=True), "value not fp16-exact"
    return h.view(np.uint16)


def bf16_bits_of(r: np.ndarray) -> np.ndarray:
    """Bit patterns of float64 values that are already exactly representable in bf16."""
    r = np.asarray(r, dtype=np.float64)
    f = r.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), r, equal_nan=True), "value not bf16-exact"
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF), "value not bf16-exact"
    return (u >> 16).astype(np.uint16)


def decode_f16(bits) -> np.ndarray:
    """fp16 bit patterns -> float64, from the binary16 field definition."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = (b >> 15) & 1
    e = (b >> 10) & 0x1F
    f = b & 0x3FF
    sign = np.where(s == 1, -1.0, 1.0)
    normal = np.ldexp((1024 + f).astype(np.float64), e - 25)   # (1 + f/2^10) * 2^(e-15)
    sub = np.ldexp(f.astype(np.float64), -24)                  # f/2^10 * 2^-14
    val = np.where(e == 0, sub, normal)
    val = np.where(e == 31, np.where(f == 0, np.inf, np.nan), val)
    return sign * val


def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (bf16 is the top half of a binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def decode_e4m3(codes) -> np.ndarray:
    """OCP E4M3 ("fn") codes -> float64.

    code = s eeee mmm: exponent field 0 gives subnormals m * 2^-9, otherwise
    (8 + m) * 2^(e - 10); 0x7F / 0xFF are NaN (must not occur in inputs).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    sign = np.where(s == 1, -1.0, 1.0)
    val = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), e - 10))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def encode_e4m3(x) -> np.ndarray:
    """float64 values -> OCP E4M3 ("fn") codes, rounding to nearest (ties to even).

    Magnitudes above 448 saturate to 448 (the format has no infinity; a writer
    that scales by amax / 448 only ever exceeds 448 by a rounding error). The
    sign is kept, also for results that round to zero (code 0x80).
    """
    x = np.asarray(x, dtype=np.float64)
    assert not np.any(np.isnan(x)), "NaN has no E4M3 code here"
    r = round_to(np.clip(x, -448.0, 448.0), E4M3)
    sign = np.signbit(r).astype(np.int64)
    a = np.abs(r)
    sub = a < 2.0 ** -6
    m_sub = np.rint(a * 2.0 ** 9).astype(np.int64)             # a = m * 2^-9, m < 8
    _, e2 = np.frexp(np.where(sub, 1.0, a))                      # a = f * 2^e2, 0.5 <= f < 1
    e = e2 - 1                                                   # a = (8 + m) * 2^(e - 3)
    m_norm = np.rint(np.where(sub, 8.0, a) / np.ldexp(1.0, e - 3)).astype(np.int64) - 8
    code = np.where(sub, m_sub, ((e + 7) << 3) | m_norm)
    return ((sign << 7) | code).astype(np.uint8)
