"""Pins of the oracle's MX quantiser (oracle/mx_quantize.py) against what the
definitions fix: exponent minimality, torch's round-to-nearest-even float8
casts, half-step round-trip error, hand-built ties, the zero / partial /
clamped block cases, scale placement read back through the GEMM oracle's
atom expansion, and the separately written quantiser of the input generator.
All on the CPU."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.mx_quantize import FMAX

E4, E5 = oracle.FMT_E4M3, oracle.FMT_E5M2
TORCH_FP8 = {E4: torch.float8_e4m3fn, E5: torch.float8_e5m2}


def spread(rng, shape):
    """float32 values whose blocks span many binades (so exponents vary widely)."""
    mag = np.ldexp(1.0, rng.integers(-30, 30, size=shape))
    return (rng.standard_normal(shape) * mag).astype(np.float32)


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("sf", [16, 32])
def test_exponent_is_smallest(fmt, sf):
    x = spread(np.random.default_rng(1), (2, 37, 160))
    bm = oracle.block_max(x, sf)
    e = oracle.block_exponent(bm, fmt)
    live = (bm > 0) & (e > -127) & (e < 127)
    assert live.sum() > 100
    assert np.all(np.ldexp(FMAX[fmt], e[live]) >= bm[live])
    assert np.all(np.ldexp(FMAX[fmt], e[live] - 1) < bm[live])


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("sf", [16, 32])
def test_codes_are_torch_rne_of_scaled_values(fmt, sf):
    x = spread(np.random.default_rng(2), (3, 50, 128))
    codes, _, e = oracle.mx_quantize(x, sf, fmt)
    q = np.ldexp(x.astype(np.float64), -np.repeat(e, sf, axis=2)[:, :, :x.shape[2]])
    assert np.all(np.abs(q) <= FMAX[fmt])
    ref = torch.from_numpy(q.astype(np.float32)).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_round_trip_within_half_step(fmt):
    x = spread(np.random.default_rng(3), (1, 64, 256))
    codes, _, e = oracle.mx_quantize(x, 32, fmt)
    per_k = np.repeat(e, 32, axis=2)
    back = np.ldexp(oracle.decode(codes, fmt), per_k)
    q = np.abs(np.ldexp(x.astype(np.float64), -per_k))
    # code step at |q|: 2^(binade - mantissa bits), floored at the subnormal step
    mbits, min_exp = (3, -6) if fmt == E4 else (2, -14)
    binade = np.floor(np.log2(np.maximum(q, np.ldexp(1.0, min_exp))))
    step = np.ldexp(1.0, (binade - mbits).astype(np.int64))
    assert np.all(np.abs(back - x) <= np.ldexp(step / 2, per_k))


def test_hand_built_ties_go_to_even():
    # one block whose max is FMAX, so e = 0 and the codes are of x itself
    cases = {
        E4: [(1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
             (-1.0625, 0xB8), (-(2.0 ** -11), 0x80), (0.0, 0x00), (-0.0, 0x80), (448.0, 0x7E)],
        E5: [(1.125, 0x3C), (1.375, 0x3E), (2.0 ** -17, 0x00), (3 * 2.0 ** -17, 0x02),
             (-1.125, 0xBC), (57344.0, 0x7B)],
    }
    for fmt, pairs in cases.items():
        row = np.zeros(32, dtype=np.float32)
        row[0] = FMAX[fmt]
        for i, (v, _) in enumerate(pairs):
            row[1 + i] = v
        codes, sf, e = oracle.mx_quantize(row[None, None, :], 32, fmt)
        assert e[0, 0, 0] == 0
        for i, (v, want) in enumerate(pairs):
            assert codes[0, 0, 1 + i] == want, (fmt, v, hex(codes[0, 0, 1 + i]), hex(want))


def test_zero_partial_and_clamped_blocks():
    x = np.zeros((1, 3, 48), dtype=np.float32)        # K = 48, sf = 32: the second block is partial
    x[0, 1, 40] = 3.0                                  # partial block of row 1: bm = 3
    x[0, 1, 5] = 1e30                                  # first block of row 1: large exponent
    x[0, 2, :32] = 1e-41                               # subnormal float32: exponent clamps at -127
    codes, sf, e = oracle.mx_quantize(x, 32, E4)
    assert e[0, 0, 0] == 0 and e[0, 0, 1] == 0          # all-zero blocks: scale byte 127
    assert np.all(codes[0, 0] == 0)
    assert e[0, 1, 1] == -7                             # 448 * 2^-8 < 3 <= 448 * 2^-7
    assert np.ldexp(448.0, int(e[0, 1, 0])) >= 1e30 > np.ldexp(448.0, int(e[0, 1, 0]) - 1)
    assert e[0, 2, 0] == -127
    assert np.all(codes[0, 2, :32] == oracle.encode_rne(np.ldexp(np.float64(np.float32(1e-41)), 127)
                                                        * np.ones(32), E4))


@pytest.mark.parametrize("sf", [16, 32])
def test_scale_placement_reads_back_through_the_gemm_oracle(sf):
    rng = np.random.default_rng(4)
    l, mn, k = 2, 200, 3 * 4 * sf + 16                 # ragged rows and a ragged last atom along K
    x = spread(rng, (l, mn, k))
    _, phys, e = oracle.mx_quantize(x, sf, E4)
    assert phys.size == 512 * l * (-(-mn // 128)) * (-(-k // (4 * sf)))
    got = oracle.sf_atom.expand_scale_bytes(phys, mn, k, l, sf)
    assert np.array_equal(np.asarray(got).reshape(e.shape), (e + 127).astype(np.uint8))
    # padding entries (rows past mn, K-blocks past ceil(k/sf)) hold 127
    lv = oracle.sf_logical_view(phys, mn, k, l, sf)
    rows = np.arange(32)[:, None, None] + 32 * np.arange(4)[None, :, None] + 128 * np.arange(lv.shape[2])[None, None, :]
    assert np.all(lv[rows >= mn] == 127)
    kbs = np.arange(4)[:, None] + 4 * np.arange(lv.shape[4])[None, :]
    assert np.all(lv[:, :, :, kbs >= -(-k // sf), :] == 127)


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("sf", [16, 32])
def test_matches_the_input_generators_quantiser(fmt, sf):
    rng = np.random.default_rng(5)
    l, mn, k = 2, 130, 4 * sf + 32
    x = spread(rng, (l, mn, k))
    codes, phys, _ = oracle.mx_quantize(x, sf, fmt)
    wcodes, wbytes = W.mx_quantize(x, sf, fmt)
    assert np.array_equal(codes, wcodes)
    assert np.array_equal(phys, W.pack_sf(wbytes, mn, k, l, sf))
