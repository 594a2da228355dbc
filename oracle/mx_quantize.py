"""MX block quantisation: float32 -> E4M3/E5M2 codes plus E8M0 block scales in the SF atom layout.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes.  "GEMM + RoPE + MXFP8 Projection (SM100)", section
"Equations", quantises with blocks of 32 elements, one E8M0 scale per block
and E4M3 data, and section "Shapes" of "GEMM + Amax (SM100)" fixes where a
(row, K-block) scale lives in the atom layout.  The pages name the
quantisation but do not spell out its scale rule.  The reading taken is the
rule the GEMM's own test configurations state for their inputs (a scale of
2^ceil(log2(blockmax / FMAX))), written without logarithms:

* blocks are sf consecutive K elements of one row (sf = 16 or 32); K
  elements past K in the last block are absent;
* bm = max |x| over the block;
* e = the smallest integer with FMAX * 2^e >= bm, clamped to [-127, 127]
  (FMAX = 448 for E4M3, 57344 for E5M2, 6 for E2M1); e = 0 when bm = 0;
* scale byte = e + 127;
* code = x * 2^-e rounded to the nearest finite code of the format, ties to
  the code with the even mantissa (the even code), sign kept (a negative
  value that rounds to zero gives the -0 code).  The choice of e makes
  |x * 2^-e| <= FMAX, so nothing saturates;
* scale bytes go to their (row, K-block) entries of the physical
  (L, ceil(MN/128), ceil(K/(4 sf)), 32, 4, 4) buffer; padding entries (rows
  past MN, K-blocks past ceil(K/sf)) hold 127 (a scale of 1).

How: exponents by an exact upward search (numpy ldexp comparisons, no
logarithm); codes by a nearest-value search over the 256-entry decode tables
of ``codecs``; scale bytes written through ``sf_atom.sf_logical_view``, the
index map the GEMM oracle reads scales with.  Values are handled in float64,
where x * 2^-e is exact.

Pins (``tests/test_oracle_quantize.py``): exponent minimality
(FMAX * 2^(e-1) < bm <= FMAX * 2^e); codes equal torch's float8 casts (a
round-to-nearest-even library routine) of the scaled values; round-trip
error at most half a code step; hand-built ties; zero, partial and clamped
blocks; scale placement read back through the GEMM oracle's expansion; and
agreement with the separately written quantiser of the input generator.
"""

import numpy as np

from .codecs import FMT_E2M1, FMT_E4M3, FMT_E5M2, decode
from .sf_atom import sf_logical_view, sf_physical_shape

FMAX = {FMT_E4M3: 448.0, FMT_E5M2: 57344.0, FMT_E2M1: 6.0}


def _cdiv(a, b):
    return -(-a // b)


def block_max(x, sf_vec_size):
    """max |x| per (l, row, K-block) of float32 x (L, rows, K), as float64 (L, rows, ceil(K/sf))."""
    x = np.asarray(x, dtype=np.float32)
    l, rows, k = x.shape
    kb = _cdiv(k, sf_vec_size)
    ax = np.zeros((l, rows, kb * sf_vec_size), dtype=np.float64)
    ax[:, :, :k] = np.abs(x.astype(np.float64))
    return ax.reshape(l, rows, kb, sf_vec_size).max(axis=3)


def block_exponent(bm, fmt):
    """Smallest integer e with FMAX * 2^e >= bm, clamped to [-127, 127]; 0 where bm == 0."""
    bm = np.asarray(bm, dtype=np.float64)
    fmax = FMAX[fmt]
    # start below the answer: with frexp exponent P, bm >= 2^(P-1), and FMAX < 2^16 gives
    # FMAX * 2^(P-17) < 2^(P-1) <= bm; then raise e one at a time while FMAX * 2^e < bm
    _, P = np.frexp(bm)
    e = (P - 17).astype(np.int64)
    for _ in range(32):  # each pass raises every unsatisfied e by one; at most 17 are needed
        low = (bm > 0) & (np.ldexp(fmax, e) < bm)
        if not low.any():
            break
        e = e + low
    assert not ((bm > 0) & (np.ldexp(fmax, e) < bm)).any()
    e = np.where(bm > 0, e, 0)
    return np.clip(e, -127, 127).astype(np.int64)


def _positive_table(fmt):
    """Finite non-negative values of the format in code order (which is value order) and their codes."""
    codes = np.arange(8 if fmt == FMT_E2M1 else 128, dtype=np.uint8)
    vals = decode(codes, fmt)
    keep = np.isfinite(vals)
    vals, codes = vals[keep], codes[keep]
    assert np.all(np.diff(vals) > 0)
    return vals, codes


def encode_rne(q, fmt):
    """Nearest finite code to float64 q (|q| <= FMAX), ties to the even code, sign kept."""
    q = np.asarray(q, dtype=np.float64)
    vals, codes = _positive_table(fmt)
    a = np.abs(q)
    assert np.all(a <= vals[-1]), "values beyond FMAX"
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    pick_hi = np.where(a == vals[hi], True, pick_hi)      # exact hits
    c = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    sign = 0x8 if fmt == FMT_E2M1 else 0x80
    return np.where(np.signbit(q), c | sign, c).astype(np.uint8)


def place_scales(scale_bytes, mn, k, l, sf_vec_size, pad_byte=127):
    """Write per-(l, row, K-block) scale bytes into a new flat physical SF buffer via the logical view."""
    mnb, kg = _cdiv(mn, 128), _cdiv(k, 4 * sf_vec_size)
    kb = _cdiv(k, sf_vec_size)
    full = np.full((l, mnb * 128, kg * 4), pad_byte, dtype=np.uint8)
    full[:, :mn, :kb] = np.asarray(scale_bytes, dtype=np.uint8).reshape(l, mn, kb)
    # full[l, 128*i2 + 32*i1 + i0, 4*i4 + i3] -> logical [i0, i1, i2, i3, i4, l]
    by_index = full.reshape(l, mnb, 4, 32, kg, 4).transpose(3, 2, 1, 5, 4, 0)
    phys = np.empty(int(np.prod(sf_physical_shape(mn, k, l, sf_vec_size))), dtype=np.uint8)
    sf_logical_view(phys, mn, k, l, sf_vec_size)[...] = by_index
    return phys


def pack_e2m1(nibbles):
    """One 4-bit code per element (..., K), K even -> packed bytes (..., K/2), element 2i low."""
    n = np.asarray(nibbles, dtype=np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def mx_quantize(x, sf_vec_size, fmt):
    """MX-quantise float32 x (L, MN, K) or (MN, K).

    Returns (codes uint8 (L, MN, K), physical SF buffer uint8 (flat), per-block
    exponents int64 (L, MN, ceil(K/sf))).  For E2M1 the codes are one 4-bit
    code per element (pack with ``pack_e2m1``).
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim == 2:
        x = x[None]
    l, mn, k = x.shape
    e = block_exponent(block_max(x, sf_vec_size), fmt)
    per_k = np.repeat(e, sf_vec_size, axis=2)[:, :, :k]
    q = np.ldexp(x.astype(np.float64), -per_k)
    codes = encode_rne(q, fmt)
    sf = place_scales((e + 127).astype(np.uint8), mn, k, l, sf_vec_size)
    return codes, sf, e
