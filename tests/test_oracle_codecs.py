"""Pins of the oracle's E4M3 / E5M2 / E8M0 decoders.

Each decoder is compared, code by code, with torch's float8 dtypes (a decoder
written independently of the oracle), and the documented special values of
the OCP 8-bit and MX formats are checked directly.
"""

import math

import numpy as np
import pytest
import torch

from oracle import codecs

ALL = np.arange(256, dtype=np.uint8)


def _torch_decode(dtype):
    return torch.from_numpy(ALL.copy()).view(dtype).double().numpy()


@pytest.mark.parametrize("fn,dtype", [
    (codecs.decode_e4m3, torch.float8_e4m3fn),
    (codecs.decode_e5m2, torch.float8_e5m2),
    (codecs.decode_e8m0, torch.float8_e8m0fnu),
])
def test_all_codes_match_torch(fn, dtype):
    ours = fn(ALL)
    ref = _torch_decode(dtype)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # signed zero as well
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_e4m3_special_values():
    d = codecs.decode_e4m3
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    assert d(0x01) == 2.0 ** -9            # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert d(0x08) == 2.0 ** -6            # smallest normal
    assert d(0x38) == 1.0
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    assert not np.isinf(codecs.E4M3_TABLE).any()   # "fn": no infinities


def test_e5m2_special_values():
    d = codecs.decode_e5m2
    assert d(0x7B) == 57344.0
    assert d(0x7C) == math.inf and d(0xFC) == -math.inf
    assert all(math.isnan(d(c)) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert d(0x01) == 2.0 ** -16
    assert d(0x04) == 2.0 ** -14
    assert d(0x3C) == 1.0


def test_e8m0_special_values():
    d = codecs.decode_e8m0
    assert d(0x7F) == 1.0
    assert d(0x00) == 2.0 ** -127
    assert d(0xFE) == 2.0 ** 127
    assert math.isnan(d(0xFF))
    # strictly increasing powers of two over the finite range
    v = codecs.E8M0_TABLE[:255]
    assert np.all(v[1:] == 2 * v[:-1])


def test_decode_dispatch():
    codes = np.array([[0x38, 0x3C]], dtype=np.uint8)
    assert codecs.decode(codes, "e4m3")[0, 0] == 1.0
    assert codecs.decode(codes, codecs.FMT_E5M2)[0, 1] == 1.0
    with pytest.raises(ValueError):
        codecs.fmt_id(7)
