"""Pins of the oracle's packed FP4 (E2M1) path: the decoder against the MX
specification's E2M1 value list, the nibble order (a reading: element 2i in
the low nibble), an exact Fraction brute force of the GEMM on packed FP4
operands (element values taken from the specification's list and scales by
the atom byte offset, independently of the oracle), the identity invariant,
and the FP4 quantiser against the input generator's separately written one
and against hand-built ties.  torch has the float4_e2m1fn_x2 dtype but no
conversion from it, so the decoder's pin is the specification's table."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W
from oracle.mx_quantize import FMAX

E2M1 = oracle.FMT_E2M1
# the MX specification's E2M1 magnitudes for codes 0..7 (codes 8..15: the same, negative)
SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def spec_value(nibble):
    v = SPEC[nibble & 7]
    return -v if nibble & 8 else v


def test_decoder_is_the_spec_table():
    got = oracle.decode_e2m1(np.arange(16))
    want = np.array([spec_value(c) for c in range(16)])
    assert np.array_equal(got, want)
    assert np.signbit(got[8]) and not np.signbit(got[0])          # 0x8 is -0
    assert got.max() == 6.0 and got[1] == 0.5                      # max normal, the subnormal
    # every E2M1 value is exactly an E4M3 value (a coarser grid of the same kind)
    e4 = oracle.decode_e4m3(np.arange(256))
    assert all(v in e4 for v in got)


def test_nibble_order_and_round_trip():
    assert list(oracle.unpack_e2m1(np.array([0x21, 0xF7], dtype=np.uint8), 4)) == [1, 2, 7, 15]
    nib = np.random.default_rng(0).integers(0, 16, size=(3, 5, 64), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_e2m1(oracle.pack_e2m1(nib), 64), nib)
    assert oracle.bytes_per_row(96, E2M1) == 48 and oracle.bytes_per_row(96, oracle.FMT_E4M3) == 96


def sf_byte(phys, mn_count, k, sf, l, mn, kb):
    mnb, kg = -(-mn_count // 128), -(-k // (4 * sf))
    atom = (l * mnb + mn // 128) * kg + kb // 4
    return int(phys[512 * atom + 16 * (mn % 32) + 4 * ((mn // 32) % 4) + kb % 4])


@pytest.mark.parametrize("m,n,k,l,sf", [(5, 7, 64, 1, 32), (4, 6, 96, 2, 32), (3, 5, 128, 1, 16)])
def test_bruteforce_exact_fp4(m, n, k, l, sf):
    rng = np.random.default_rng(m + n + k)
    a = rng.integers(0, 256, size=(l, m, k // 2), dtype=np.uint8)
    b = rng.integers(0, 256, size=(l, n, k // 2), dtype=np.uint8)
    sfa = rng.integers(117, 138, size=oracle.sf_physical_shape(m, k, l, sf), dtype=np.uint8).reshape(-1)
    sfb = rng.integers(117, 138, size=oracle.sf_physical_shape(n, k, l, sf), dtype=np.uint8).reshape(-1)
    c, s, amax = oracle.gemm_amax(a, b, sfa, sfb, m, n, k, l, sf, E2M1, E2M1)

    def elem(buf, bi, r, kk):          # byte kk // 2, low nibble for even kk
        byte = int(buf[bi, r, kk // 2])
        return spec_value(byte & 0xF if kk % 2 == 0 else byte >> 4)

    for bi in range(l):
        for i in range(m):
            for j in range(n):
                acc = Fraction(0)
                for kk in range(k):
                    e = sf_byte(sfa, m, k, sf, bi, i, kk // sf) + sf_byte(sfb, n, k, sf, bi, j, kk // sf) - 254
                    acc += Fraction(elem(a, bi, i, kk)) * Fraction(elem(b, bi, j, kk)) * Fraction(2) ** e
                assert Fraction(float(c[bi, i, j])) == acc    # few terms of short significands: exact


def test_identity_fp4_reproduces_b():
    m = k = 64
    n = 40
    nib = np.zeros((1, m, k), np.uint8)
    nib[0, np.arange(m), np.arange(k)] = 0x2                      # 1.0 in E2M1
    a = oracle.pack_e2m1(nib)
    b = np.random.default_rng(3).integers(0, 256, size=(1, n, k // 2), dtype=np.uint8)
    sfa = np.full(oracle.sf_physical_shape(m, k, 1, 32), 127, np.uint8).reshape(-1)
    sfb = np.random.default_rng(4).integers(120, 135, size=oracle.sf_physical_shape(n, k, 1, 32),
                                            dtype=np.uint8).reshape(-1)
    c, _, _ = oracle.gemm_amax(a, b, sfa, sfb, m, n, k, 1, 32, E2M1, E2M1)
    bh = oracle.dequantize(b, E2M1, sfb, n, k, 1, 32)
    assert np.array_equal(c[0], bh[0].T)


def test_fp4_quantiser_ties_and_minimality():
    row = np.zeros(32, dtype=np.float32)
    row[0] = 6.0                                                   # e = 0: codes of x itself
    vals = [1.75, 0.75, 5.0, 0.25, -1.25, 2.5, 3.5, -0.1]
    want = [0x4, 0x2, 0x6, 0x0, 0xA, 0x4, 0x6, 0x8]                # ties to the even code; -0.1 -> -0
    row[1:1 + len(vals)] = vals
    codes, _, e = oracle.mx_quantize(row[None, None, :], 32, E2M1)
    assert e[0, 0, 0] == 0
    assert list(codes[0, 0, 1:1 + len(vals)]) == want
    x = (np.random.default_rng(5).standard_normal((1, 40, 128)) *
         np.ldexp(1.0, np.random.default_rng(6).integers(-20, 20, size=(1, 40, 128)))).astype(np.float32)
    bm = oracle.block_max(x, 32)
    e = oracle.block_exponent(bm, E2M1)
    live = (bm > 0) & (e > -127) & (e < 127)
    assert np.all(np.ldexp(FMAX[E2M1], e[live]) >= bm[live])
    assert np.all(np.ldexp(FMAX[E2M1], e[live] - 1) < bm[live])


@pytest.mark.parametrize("sf", [16, 32])
def test_fp4_quantiser_matches_the_input_generator(sf):
    x = np.random.default_rng(8).standard_normal((2, 70, 192)).astype(np.float32)
    codes, phys, _ = oracle.mx_quantize(x, sf, E2M1)
    wcodes, wbytes = W.mx_quantize(x, sf, E2M1)
    assert np.array_equal(oracle.pack_e2m1(codes), wcodes)
    assert np.array_equal(phys, W.pack_sf(wbytes, 70, 192, 2, sf))
