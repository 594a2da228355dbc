"""Expansion of the scale-factor atom layout into one scale per (row, K-block).

TEST INFRASTRUCTURE ONLY (see the package docstring).

"GEMM + Amax (SM100)", section "Shapes" gives the logical SF shape
``(32, 4, ceil(MN/128), 4, ceil(K/(4*sf)), L)`` and section "Parameters" names
its modes ``(ATOM_M0, ATOM_M1, rest_M, ATOM_K, rest_K, L)``.  Section "Using
JAX arrays" states that the physical C-contiguous allocation is
``(L, ceil(MN/128), ceil(K/(4*sf)), 32, 4, 4)`` and that the logical view is
that allocation permuted by ``(3, 4, 1, 5, 2, 0)``.

Reading (the pages name the modes but do not say which index is which row
or K-block): the first-listed sub-mode varies fastest, so logical index
``(i0, i1, i2, i3, i4, l)`` holds the scale of

    row     mn = i0 + 32*i1 + 128*i2
    K-block kb = i3 + 4*i4          (K elements [kb*sf, (kb+1)*sf))

Rows >= MN of the last 128-row group and K-blocks >= ceil(K/sf) of the last
group are padding and are never read here.

This module builds the logical view with a reshape + transpose of the
physical buffer and then gathers with the index formulas above.  It does not
use a byte-offset formula.

Pins (``tests/test_oracle_sf_atom.py``): the physical shape of the worked
JAX example on the page (m=512, k=256, sf=32 -> (1, 4, 2, 32, 4, 4)); the
permutation maps the physical shape onto the logical one; a single poked
logical entry changes exactly rows i0+32*i1+128*i2 and K range
[sf*(i3+4*i4), +sf) of the expansion.  Against the vendor library's own
convention the row/K assignment is parity unpinned (the pages give no
non-uniform-scale example).
"""

import numpy as np

from .codecs import decode_e8m0


def _cdiv(a, b):
    return -(-a // b)


def sf_physical_shape(mn, k, l, sf_vec_size):
    """Physical C-contiguous SF shape (L, ceil(MN/128), ceil(K/(4 sf)), 32, 4, 4)."""
    return (l, _cdiv(mn, 128), _cdiv(k, 4 * sf_vec_size), 32, 4, 4)


def sf_logical_shape(mn, k, l, sf_vec_size):
    """Logical SF shape (32, 4, ceil(MN/128), 4, ceil(K/(4 sf)), L)."""
    return (32, 4, _cdiv(mn, 128), 4, _cdiv(k, 4 * sf_vec_size), l)


def sf_logical_view(phys, mn, k, l, sf_vec_size):
    """View a physical SF buffer (any shape with the right byte count) as the logical 6-D tensor."""
    shape = sf_physical_shape(mn, k, l, sf_vec_size)
    return np.asarray(phys, dtype=np.uint8).reshape(shape).transpose(3, 4, 1, 5, 2, 0)


def expand_scale_bytes(phys, mn, k, l, sf_vec_size):
    """E8M0 byte for every (batch, row, K-block): uint8 array (L, MN, ceil(K/sf))."""
    lv = sf_logical_view(phys, mn, k, l, sf_vec_size)
    kb_count = _cdiv(k, sf_vec_size)
    rows = np.arange(mn)
    kbs = np.arange(kb_count)
    i0 = (rows % 32)[:, None]
    i1 = ((rows // 32) % 4)[:, None]
    i2 = (rows // 128)[:, None]
    i3 = (kbs % 4)[None, :]
    i4 = (kbs // 4)[None, :]
    out = np.empty((l, mn, kb_count), dtype=np.uint8)
    for b in range(l):
        out[b] = lv[i0, i1, i2, i3, i4, b]
    return out


def expand_scales(phys, mn, k, l, sf_vec_size):
    """Scale value 2^(byte-127) for every (batch, row, K-block): float64 (L, MN, ceil(K/sf))."""
    return decode_e8m0(expand_scale_bytes(phys, mn, k, l, sf_vec_size))
