"""Pins of the oracle's scale-factor atom expansion.

* Shapes: the page's worked example (tests/golden/worked_example.json) fixes
  the physical shape; the page's permutation (3, 4, 1, 5, 2, 0) must turn it
  into the logical shape of section "Shapes".
* Index map: one poked logical entry (i0, i1, i2, i3, i4, l) must change the
  expanded scale of exactly row i0 + 32*i1 + 128*i2, K-block i3 + 4*i4,
  batch l -- and nothing else (the reading documented in oracle/sf_atom.py).
* Padding entries are never read.
"""

import json
import os

import numpy as np
import pytest

from oracle import sf_atom

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def test_worked_example_shapes():
    g = json.load(open(GOLDEN))
    m, n, k, l, sf = g["m"], g["n"], g["k"], g["l"], g["sf_vec_size"]
    assert list(sf_atom.sf_physical_shape(m, k, l, sf)) == g["sfa_physical_shape"]
    assert list(sf_atom.sf_physical_shape(n, k, l, sf)) == g["sfb_physical_shape"]
    assert list(sf_atom.sf_logical_shape(m, k, l, sf)) == g["sfa_logical_shape"]
    assert list(sf_atom.sf_logical_shape(n, k, l, sf)) == g["sfb_logical_shape"]
    perm = g["physical_to_logical_permutation"]
    phys = np.zeros(g["sfa_physical_shape"], dtype=np.uint8)
    assert list(phys.transpose(perm).shape) == g["sfa_logical_shape"]
    lv = sf_atom.sf_logical_view(phys.reshape(-1), m, k, l, sf)
    assert list(lv.shape) == g["sfa_logical_shape"]


@pytest.mark.parametrize("mn,k,l,sf", [(128, 128, 1, 32), (300, 592, 2, 32), (257, 200, 3, 16),
                                        (4000, 2048, 1, 16)])
def test_buffer_size_closed_form(mn, k, l, sf):
    shape = sf_atom.sf_physical_shape(mn, k, l, sf)
    assert int(np.prod(shape)) == 512 * l * (-(-mn // 128)) * (-(-k // (4 * sf)))


@pytest.mark.parametrize("mn,k,l,sf", [(256, 256, 1, 32), (300, 592, 2, 32), (257, 200, 2, 16)])
def test_single_poke_hits_one_row_and_block(mn, k, l, sf):
    rng = np.random.default_rng(0)
    shape = sf_atom.sf_physical_shape(mn, k, l, sf)
    kb_count = -(-k // sf)
    for _ in range(40):
        # choose an in-range (row, K-block, batch) and derive its logical index
        row = int(rng.integers(0, mn))
        kb = int(rng.integers(0, kb_count))
        b = int(rng.integers(0, l))
        i0, i1, i2 = row % 32, (row // 32) % 4, row // 128
        i3, i4 = kb % 4, kb // 4
        phys = np.full(shape, 127, dtype=np.uint8)
        lv = phys.transpose(3, 4, 1, 5, 2, 0)       # a writable view onto phys
        lv[i0, i1, i2, i3, i4, b] = 133
        got = sf_atom.expand_scale_bytes(phys.reshape(-1), mn, k, l, sf)
        changed = np.argwhere(got != 127)
        assert changed.tolist() == [[b, row, kb]]
        assert sf_atom.expand_scales(phys.reshape(-1), mn, k, l, sf)[b, row, kb] == 2.0 ** 6


def test_padding_entries_ignored():
    mn, k, l, sf = 130, 80, 1, 32        # rows 130..255 and K-blocks 3..3 are padding
    shape = sf_atom.sf_physical_shape(mn, k, l, sf)
    phys = np.full(shape, 127, dtype=np.uint8)
    lv = phys.transpose(3, 4, 1, 5, 2, 0)
    lv[5, 0, 1, :, 0, 0] = 0xFF            # row 133 (past MN)
    lv[:, :, :, 3, 0, 0] = 0xFF            # K-block 3 (past ceil(80/32) = 3 blocks)
    got = sf_atom.expand_scale_bytes(phys.reshape(-1), mn, k, l, sf)
    assert got.shape == (1, 130, 3)
    assert np.all(got == 127)
