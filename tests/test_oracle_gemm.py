"""Pins of the oracle's dequantise + contract + amax.

* Exact brute force: on tiny shapes, values decoded by torch's float8 dtypes
  and scales looked up by the byte offset 16*(mn%32) + 4*((mn//32)%4) + kb%4
  inside atom (l, mn//128, kb//4) are summed as exact rationals
  (fractions.Fraction).  The fp64 oracle must agree within K*2^-53*S.
* Unit scales (the page's worked example, all E8M0 bytes 127): C equals
  torch.matmul of torch-decoded operands.
* Identity operand: A = I (E4M3 code 0x38 = 1.0), unit scales => C = B_hat^T.
* Scale doubling: +1 on one SFA byte changes C by exactly that block's
  partial sum, in exactly the rows that byte covers.
* Sign flip / operand swap / K-block permutation symmetries.
* Amax closed form, NaN propagation, empty output.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import gemm_amax as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")

E4M3, E5M2 = 0, 1
TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def cdiv(a, b):
    return -(-a // b)


def finite_codes(rng, shape, fmt):
    """Random element codes excluding NaN / inf."""
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    if fmt == E4M3:
        bad = (c & 0x7F) == 0x7F
    else:
        bad = (c & 0x7C) == 0x7C
    c[bad] = 0x30
    return c


def random_phys_sf(rng, mn, k, l, sf, lo=117, hi=137):
    shape = oracle.sf_physical_shape(mn, k, l, sf)
    return rng.integers(lo, hi + 1, size=shape, dtype=np.uint8).reshape(-1)


def torch_decode(codes, fmt):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(TORCH_DT[fmt]).double().numpy()


def sf_byte_by_offset(phys, mn_count, k, sf, l, mn, kb):
    """Independent lookup of one scale byte through the atom byte offset."""
    mnb = cdiv(mn_count, 128)
    kg = cdiv(k, 4 * sf)
    atom = (l * mnb + mn // 128) * kg + kb // 4
    return int(phys[512 * atom + 16 * (mn % 32) + 4 * ((mn // 32) % 4) + kb % 4])


def exact_reference(a, b, sfa, sfb, m, n, k, l, sf, a_fmt, b_fmt):
    av = torch_decode(a, a_fmt)
    bv = torch_decode(b, b_fmt)
    c = [[[None] * n for _ in range(m)] for _ in range(l)]
    s = [[[None] * n for _ in range(m)] for _ in range(l)]
    for bi in range(l):
        for i in range(m):
            for j in range(n):
                acc = Fraction(0)
                mag = Fraction(0)
                for kk in range(k):
                    ea = sf_byte_by_offset(sfa, m, k, sf, bi, i, kk // sf) - 127
                    eb = sf_byte_by_offset(sfb, n, k, sf, bi, j, kk // sf) - 127
                    p = Fraction(float(av[bi, i, kk])) * Fraction(float(bv[bi, j, kk])) \
                        * Fraction(2) ** (ea + eb)
                    acc += p
                    mag += abs(p)
                c[bi][i][j] = acc
                s[bi][i][j] = mag
    return c, s


@pytest.mark.parametrize("m,n,k,l,sf,af,bf", [
    (5, 7, 32, 1, 32, E4M3, E4M3),
    (8, 3, 64, 2, 16, E5M2, E4M3),
    (4, 6, 96, 1, 32, E4M3, E5M2),
    (3, 5, 48, 1, 32, E5M2, E5M2),     # K % sf != 0: a partial last block
    (6, 4, 80, 1, 16, E4M3, E4M3),
])
def test_bruteforce_exact(m, n, k, l, sf, af, bf):
    rng = np.random.default_rng(m * 1000 + n * 10 + k)
    a = finite_codes(rng, (l, m, k), af)
    b = finite_codes(rng, (l, n, k), bf)
    sfa = random_phys_sf(rng, m, k, l, sf)
    sfb = random_phys_sf(rng, n, k, l, sf)
    c, s, amax = oracle.gemm_amax(a, b, sfa, sfb, m, n, k, l, sf, af, bf)
    c_ex, s_ex = exact_reference(a, b, sfa, sfb, m, n, k, l, sf, af, bf)
    for bi in range(l):
        for i in range(m):
            for j in range(n):
                bound = float(s_ex[bi][i][j]) * k * 2.0 ** -53
                assert abs(Fraction(float(c[bi, i, j])) - c_ex[bi][i][j]) <= Fraction(bound)
                assert abs(s[bi, i, j] - float(s_ex[bi][i][j])) <= bound
    ex_amax = max(abs(v) for plane in c_ex for row in plane for v in row)
    assert abs(Fraction(amax) - ex_amax) <= Fraction(float(ex_amax) * k * 2.0 ** -52)
    # the scalar-loop form agrees with the matmul form
    c2, s2, amax2 = oracle.gemm_amax_loops(a, b, sfa, sfb, m, n, k, l, sf, af, bf)
    np.testing.assert_allclose(c2, c, rtol=0, atol=1e-12 * np.max(s))


def test_worked_example_unit_scales():
    g = json.load(open(GOLDEN))
    m, n, k, l, sf = g["m"], g["n"], g["k"], g["l"], g["sf_vec_size"]
    rng = np.random.default_rng(1)
    a = finite_codes(rng, (l, m, k), E5M2)
    b = finite_codes(rng, (l, n, k), E5M2)
    sfa = np.full(oracle.sf_physical_shape(m, k, l, sf), g["scale_byte"], np.uint8).reshape(-1)
    sfb = np.full(oracle.sf_physical_shape(n, k, l, sf), g["scale_byte"], np.uint8).reshape(-1)
    c, _, amax = oracle.gemm_amax(a, b, sfa, sfb, m, n, k, l, sf, E5M2, E5M2)
    ta = torch.from_numpy(torch_decode(a, E5M2))
    tb = torch.from_numpy(torch_decode(b, E5M2))
    ref = torch.matmul(ta, tb.transpose(1, 2).contiguous()).numpy()
    s = np.abs(ta.numpy()) @ np.abs(tb.numpy()).transpose(0, 2, 1)
    assert np.all(np.abs(c - ref) <= 4 * k * 2.0 ** -53 * s)
    assert amax == pytest.approx(float(np.max(np.abs(ref))), rel=1e-12)


def test_identity_operand_reproduces_b():
    m = k = 64
    n = 96
    rng = np.random.default_rng(2)
    a = np.zeros((1, m, k), np.uint8)
    a[0, np.arange(m), np.arange(k)] = 0x38            # 1.0 in E4M3
    b = finite_codes(rng, (1, n, k), E4M3)
    sfa = np.full(oracle.sf_physical_shape(m, k, 1, 32), 127, np.uint8).reshape(-1)
    sfb = random_phys_sf(rng, n, k, 1, 32)
    c, _, _ = oracle.gemm_amax(a, b, sfa, sfb, m, n, k, 1, 32, E4M3, E4M3)
    bh = oracle.dequantize(b, E4M3, sfb, n, k, 1, 32)
    assert np.array_equal(c[0], bh[0].T)


@pytest.mark.parametrize("sf", [16, 32])
def test_scale_doubling_changes_one_block(sf):
    m, n, k, l = 300, 70, 256, 2
    rng = np.random.default_rng(3)
    a = finite_codes(rng, (l, m, k), E4M3)
    b = finite_codes(rng, (l, n, k), E4M3)
    sfa = random_phys_sf(rng, m, k, l, sf)
    sfb = random_phys_sf(rng, n, k, l, sf)
    c0, _, _ = oracle.gemm_amax(a, b, sfa, sfb, m, n, k, l, sf, E4M3, E4M3)
    for row, kb, bi in [(0, 0, 0), (37, 1, 1), (131, cdiv(k, sf) - 1, 0), (299, 2, 1)]:
        sfa2 = sfa.copy()
        mnb, kg = cdiv(m, 128), cdiv(k, 4 * sf)
        off = 512 * ((bi * mnb + row // 128) * kg + kb // 4) + 16 * (row % 32) + 4 * ((row // 32) % 4) + kb % 4
        sfa2[off] += 1
        c1, _, _ = oracle.gemm_amax(a, b, sfa2, sfb, m, n, k, l, sf, E4M3, E4M3)
        diff = c1 - c0
        # partial sum of that block, computed with the (unchanged) scales
        ah = oracle.dequantize(a, E4M3, sfa, m, k, l, sf)
        bh = oracle.dequantize(b, E4M3, sfb, n, k, l, sf)
        ks = slice(kb * sf, min(k, (kb + 1) * sf))
        part = ah[bi, row, ks] @ bh[bi, :, ks].T
        mask = np.zeros_like(diff, dtype=bool)
        mask[bi, row, :] = True
        assert np.all(diff[~mask] == 0)
        s_row = np.abs(ah[bi, row]) @ np.abs(bh[bi]).T
        assert np.all(np.abs(diff[bi, row] - part) <= 4 * k * 2.0 ** -53 * 2 * s_row)


def test_sign_flip_and_swap_and_block_permutation():
    m, n, k, l, sf = 40, 56, 192, 2, 32
    rng = np.random.default_rng(4)
    a = finite_codes(rng, (l, m, k), E4M3)
    b = finite_codes(rng, (l, n, k), E5M2)
    sfa = random_phys_sf(rng, m, k, l, sf)
    sfb = random_phys_sf(rng, n, k, l, sf)
    c, s, amax = oracle.gemm_amax(a, b, sfa, sfb, m, n, k, l, sf, E4M3, E5M2)
    tol = 4 * k * 2.0 ** -53 * s
    # sign flip of every A code
    cn, _, amax_n = oracle.gemm_amax(a ^ 0x80, b, sfa, sfb, m, n, k, l, sf, E4M3, E5M2)
    assert np.all(np.abs(cn + c) <= tol) and amax_n == pytest.approx(amax, rel=1e-13)
    # swapping (A, SFA) with (B, SFB) transposes C
    ct, _, _ = oracle.gemm_amax(b, a, sfb, sfa, n, m, k, l, sf, E5M2, E4M3)
    assert np.all(np.abs(ct.transpose(0, 2, 1) - c) <= tol)
    # permuting K-blocks identically in A, B and both scale sets leaves C unchanged
    kb = k // sf
    perm = rng.permutation(kb)
    kperm = (perm[:, None] * sf + np.arange(sf)[None, :]).reshape(-1)
    sa = oracle.sf_atom.expand_scale_bytes(sfa, m, k, l, sf)[:, :, perm]
    sb = oracle.sf_atom.expand_scale_bytes(sfb, n, k, l, sf)[:, :, perm]

    def repack(bytes_, mn):
        mnb, kg = cdiv(mn, 128), cdiv(k, 4 * sf)
        out = np.full(oracle.sf_physical_shape(mn, k, l, sf), 127, np.uint8)
        lv = out.transpose(3, 4, 1, 5, 2, 0)
        for bi in range(l):
            for r in range(mn):
                for q in range(kb):
                    lv[r % 32, (r // 32) % 4, r // 128, q % 4, q // 4, bi] = bytes_[bi, r, q]
        return out.reshape(-1)

    cp, _, _ = oracle.gemm_amax(a[:, :, kperm], b[:, :, kperm], repack(sa, m), repack(sb, n),
                                m, n, k, l, sf, E4M3, E5M2)
    assert np.all(np.abs(cp - c) <= tol)


def test_amax_closed_form_nan_and_empty():
    c = np.array([[[1.0, -7.5], [3.0, 2.0]]])
    assert oracle.amax_of(c) == 7.5
    c[0, 1, 1] = np.nan
    assert np.isnan(oracle.amax_of(c))
    assert oracle.amax_of(np.zeros((0, 4, 4))) == 0.0


def test_sampled_forms_match_full():
    m, n, k, l, sf = 150, 90, 160, 2, 16
    rng = np.random.default_rng(5)
    a = finite_codes(rng, (l, m, k), E5M2)
    b = finite_codes(rng, (l, n, k), E4M3)
    sfa = random_phys_sf(rng, m, k, l, sf)
    sfb = random_phys_sf(rng, n, k, l, sf)
    c, s, _ = oracle.gemm_amax(a, b, sfa, sfb, m, n, k, l, sf, E5M2, E4M3)
    rows = np.array([0, 33, 149])
    cr, sr = oracle.gemm_rows(a, b, sfa, sfb, m, n, k, l, sf, E5M2, E4M3, 1, rows)
    assert np.allclose(cr, c[1, rows], rtol=0, atol=1e-12 * s.max())
    il = rng.integers(0, l, 50)
    im = rng.integers(0, m, 50)
    jn = rng.integers(0, n, 50)
    ce, se = oracle.gemm_entries(a, b, sfa, sfb, m, n, k, l, sf, E5M2, E4M3, il, im, jn)
    assert np.allclose(ce, c[il, im, jn], rtol=0, atol=1e-12 * s.max())
    assert np.allclose(se, s[il, im, jn], rtol=1e-12)


def test_row_blocks_cover_every_output():
    # tiny: against the plain scalar loops (no matmul); ragged blocks of 3 rows over 2 batches
    m, n, k, l, sf = 7, 5, 64, 2, 32
    rng = np.random.default_rng(6)
    a = finite_codes(rng, (l, m, k), E4M3)
    b = finite_codes(rng, (l, n, k), E5M2)
    sfa = random_phys_sf(rng, m, k, l, sf)
    sfb = random_phys_sf(rng, n, k, l, sf)
    c_loop, s_loop, _ = oracle.gemm_amax_loops(a, b, sfa, sfb, m, n, k, l, sf, E4M3, E5M2)
    seen = np.zeros((l, m), dtype=int)
    for batch, r0, cb, sb in oracle.gemm_row_blocks(a, b, sfa, sfb, m, n, k, l, sf, E4M3, E5M2, block_rows=3):
        r1 = r0 + cb.shape[0]
        seen[batch, r0:r1] += 1
        assert cb.shape == (r1 - r0, n) and sb.shape == cb.shape
        assert np.all(np.abs(cb - c_loop[batch, r0:r1]) <= k * 2.0 ** -53 * s_loop[batch, r0:r1])
        assert np.allclose(sb, s_loop[batch, r0:r1], rtol=k * 2.0 ** -53, atol=0)
    assert np.all(seen == 1), "every row of every batch exactly once"
    # medium, sf = 16, rows not a multiple of the block: against the full oracle
    m, n, k, l, sf = 150, 90, 160, 2, 16
    a = finite_codes(rng, (l, m, k), E5M2)
    b = finite_codes(rng, (l, n, k), E4M3)
    sfa = random_phys_sf(rng, m, k, l, sf)
    sfb = random_phys_sf(rng, n, k, l, sf)
    c, s, _ = oracle.gemm_amax(a, b, sfa, sfb, m, n, k, l, sf, E5M2, E4M3)
    got_c = np.full_like(c, np.nan)
    got_s = np.full_like(s, np.nan)
    for batch, r0, cb, sb in oracle.gemm_row_blocks(a, b, sfa, sfb, m, n, k, l, sf, E5M2, E4M3, block_rows=64):
        got_c[batch, r0:r0 + cb.shape[0]] = cb
        got_s[batch, r0:r0 + cb.shape[0]] = sb
    assert np.all(np.abs(got_c - c) <= 2 * k * 2.0 ** -53 * s)
    assert np.allclose(got_s, s, rtol=2 * k * 2.0 ** -53, atol=0)

