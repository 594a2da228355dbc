"""Properties of the seeded input generator (the MX quantisation recipe and SF packing).

These check the inputs, not the GEMM: the per-block exponent is the minimal
one, the codes round to nearest with ties to even and saturate, padding SF
bytes carry the requested filler, and the generator is deterministic.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def test_exponent_is_minimal():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((2, 33, 96)) * np.exp2(rng.uniform(-20, 20, (2, 33, 1)))).astype(np.float32)
    for fmt in (W.FMT_E4M3, W.FMT_E5M2):
        e = W.block_exponents(x, 32, fmt).astype(np.float64)
        bm = np.abs(x).reshape(2, 33, 3, 32).max(axis=3).astype(np.float64)
        fmax = W.FMAX[fmt]
        assert np.all(fmax * np.exp2(e) >= bm)
        assert np.all(fmax * np.exp2(e - 1) < bm)


def test_exact_powers_and_zero_blocks():
    x = np.zeros((1, 3, 32), np.float32)
    x[0, 0, 5] = 448.0            # exactly FMAX -> e = 0
    x[0, 1, 7] = -896.0           # 2*FMAX -> e = 1
    e = W.block_exponents(x, 32, W.FMT_E4M3)
    assert e[0, :, 0].tolist() == [0, 1, 0]      # zero block -> e = 0 (byte 127)


def test_ties_to_even_and_saturation():
    # values already in code units (block max forces e = 0 via the 448 entry)
    vals = np.array([448.0, 1.0 + 1 / 16, 1.0 + 3 / 16, 3 * 2.0 ** -10, -(1.0 + 1 / 16)] + [0.0] * 27,
                    dtype=np.float32).reshape(1, 1, 32)
    codes, sb = W.mx_quantize(vals, 32, W.FMT_E4M3)
    assert sb[0, 0, 0] == 127
    dec = oracle.decode_e4m3(codes[0, 0, :5])
    # 1+1/16 is halfway between 1 and 1.125 -> even mantissa (1.0); 1+3/16 -> 1.25
    assert dec.tolist() == [448.0, 1.0, 1.25, 2 * 2.0 ** -9, -1.0]
    # saturation: the recipe never emits NaN/inf codes even at the block maximum
    big = np.full((1, 1, 32), 57344.0, np.float32)
    c5, _ = W.mx_quantize(big, 32, W.FMT_E5M2)
    assert np.all(c5 == 0x7B)


def test_round_trip_error_half_ulp():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 64, 128)).astype(np.float32)
    codes, sb = W.mx_quantize(x, 32, W.FMT_E4M3)
    e = sb.astype(np.int64) - 127
    q = oracle.decode_e4m3(codes) * np.exp2(np.repeat(e, 32, axis=2))
    # E4M3 spacing at |v| in [2^p, 2^(p+1)) is 2^(p-3); subnormal spacing 2^-9 (times 2^e)
    v = np.abs(x.astype(np.float64)) * np.exp2(-np.repeat(e, 32, axis=2))
    p = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    ulp = np.exp2(p - 3) * np.exp2(np.repeat(e, 32, axis=2))
    assert np.all(np.abs(q - x) <= 0.5 * ulp + 1e-300)


def test_pack_and_oracle_expand_agree_and_padding():
    rng = np.random.default_rng(2)
    mn, k, l, sf = 200, 320, 2, 16
    kb = -(-k // sf)
    sb = rng.integers(100, 150, (l, mn, kb), dtype=np.uint8)
    phys = W.pack_sf(sb, mn, k, l, sf, pad_byte=0xFF)
    assert phys.size == W.sf_bytes(mn, k, l, sf)
    assert np.array_equal(oracle.sf_atom.expand_scale_bytes(phys, mn, k, l, sf), sb)
    # every byte not in the expansion is padding
    assert int((phys == 0xFF).sum()) == phys.size - sb.size


def test_workload_shapes_and_determinism():
    p1 = W.make_workload(1)
    p2 = W.make_workload(1)
    assert p1["A"].shape == (1, 256, 256) and p1["SFA"].size == W.sf_bytes(256, 256, 1, 32)
    assert np.array_equal(p1["A"], p2["A"]) and np.array_equal(p1["SFB"], p2["SFB"])


def test_workload_algorithmic_counts():
    assert W.flops(8192, 24576, 1536, 1) == 618475290624
    assert W.algorithmic_bytes(8192, 24576, 1536, 1, 32) == 857210884
    assert W.algorithmic_bytes(256, 256, 256, 1, 32) == 397316
