"""Bit-exact decoders for the 8-bit formats of the GEMM + Amax inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages ("GEMM + Amax (SM100)", section "Parameters", input tensors A/B and
SFA/SFB) name the element dtypes ``float8_e4m3fn`` and ``float8_e5m2`` and the
scale dtype ``float8_e8m0fnu`` (``int8`` read as the same byte) but do not
define them.  The definitions used here are the OCP 8-bit floating point and
Microscaling (MX) format definitions those dtype names refer to:

* E4M3 ("fn": finite, no infinities): sign, 4 exponent bits (bias 7),
  3 mantissa bits.  Exponent field 0 is subnormal; the all-ones exponent with
  all-ones mantissa (codes 0x7F, 0xFF) is NaN; largest finite value 448.
* E5M2 (IEEE-like): sign, 5 exponent bits (bias 15), 2 mantissa bits.
  Exponent field 31 is +-inf (mantissa 0) or NaN; largest finite 57344.
* E8M0 (unsigned exponent): value 2^(byte - 127); byte 255 is NaN; no sign,
  no zero.

* E2M1 (packed FP4, two per byte): sign, 2 exponent bits (bias 1), 1
  mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no inf or NaN.

Each decoder is a float64 table (256 entries; 16 for E2M1) built one code at
a time from these bit fields; every entry is exact in float64.

Pins: ``tests/test_oracle_codecs.py`` compares all 256 codes of each format
with torch's own float8 dtypes (an independent library decoder) and checks
the documented special values.
"""

import math

import numpy as np

FMT_E4M3 = 0
FMT_E5M2 = 1
FMT_E2M1 = 2

_FMT_NAMES = {"e4m3": FMT_E4M3, "float8_e4m3fn": FMT_E4M3,
              "e5m2": FMT_E5M2, "float8_e5m2": FMT_E5M2,
              "e2m1": FMT_E2M1, "float4_e2m1fn_x2": FMT_E2M1}


def _e4m3(code):
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        # subnormal: 0.man * 2^(1 - bias) = man/8 * 2^-6
        return sign * math.ldexp(man, -9)
    # normal: 1.man * 2^(exp - bias) = (8 + man)/8 * 2^(exp - 7)
    return sign * math.ldexp(8 + man, exp - 10)


def _e5m2(code):
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 2) & 0x1F
    man = code & 0x3
    if exp == 0x1F:
        return sign * math.inf if man == 0 else math.nan
    if exp == 0:
        # subnormal: man/4 * 2^(1 - 15)
        return sign * math.ldexp(man, -16)
    # normal: (4 + man)/4 * 2^(exp - 15)
    return sign * math.ldexp(4 + man, exp - 17)


def _e2m1(code):
    # 4-bit: sign, 2 exponent bits (bias 1), 1 mantissa bit; no inf or NaN
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        # subnormal: man/2 * 2^(1 - 1)
        return sign * math.ldexp(man, -1)
    # normal: (2 + man)/2 * 2^(exp - 1)
    return sign * math.ldexp(2 + man, exp - 2)


def _e8m0(code):
    if code == 0xFF:
        return math.nan
    return math.ldexp(1.0, code - 127)


E4M3_TABLE = np.array([_e4m3(c) for c in range(256)], dtype=np.float64)
E5M2_TABLE = np.array([_e5m2(c) for c in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([_e8m0(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([_e2m1(c) for c in range(16)], dtype=np.float64)


def fmt_id(fmt):
    """Map a format name or id to FMT_E4M3 / FMT_E5M2."""
    if isinstance(fmt, str):
        return _FMT_NAMES[fmt.lower()]
    if fmt in (FMT_E4M3, FMT_E5M2, FMT_E2M1):
        return int(fmt)
    raise ValueError(f"unknown element format {fmt!r}")


def decode_e4m3(codes):
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_e5m2(codes):
    return E5M2_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_e8m0(codes):
    return E8M0_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_e2m1(nibbles):
    return E2M1_TABLE[np.asarray(nibbles, dtype=np.uint8) & 0xF]


def unpack_e2m1(packed, k):
    """Packed E2M1 bytes (..., ceil(k/2)) -> one 4-bit code per element (..., k).

    Reading (the pages call the container "packed fp4x2" without fixing the
    order): element 2i is the low nibble of byte i, element 2i+1 the high one."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out[..., :k]


def bytes_per_row(k, fmt):
    """Bytes of one operand row of K elements: K for the 8-bit formats, K/2 for packed E2M1."""
    return (k + 1) // 2 if fmt_id(fmt) == FMT_E2M1 else k


def element_codes(codes, fmt, rows, k, l):
    """Per-element codes (L, rows, K) of an operand buffer (L, rows, bytes_per_row(K))."""
    c = np.asarray(codes, dtype=np.uint8).reshape(l, rows, bytes_per_row(k, fmt))
    return unpack_e2m1(c, k) if fmt_id(fmt) == FMT_E2M1 else c


def decode(codes, fmt):
    """Decode per-element codes of format ``fmt`` (E4M3, E5M2, or E2M1 nibbles) to float64."""
    f = fmt_id(fmt)
    if f == FMT_E2M1:
        return decode_e2m1(codes)
    return decode_e4m3(codes) if f == FMT_E4M3 else decode_e5m2(codes)
