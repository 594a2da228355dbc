"""Dequantisation, fp64 contraction and amax of the block-scaled GEMM.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"GEMM + Amax (SM100)", section "Equations": each element is dequantised with
the scale of its group of ``sf_vec_size`` consecutive K elements, C is the
sum over K of the dequantised products (FP32 accumulation on the device,
section "Parameters", ``acc_dtype``), and Amax is the maximum of |C| over all
of m, n, l (section "Diagram": "reduce: Amax = max |C|").

Layouts follow section "Parameters": A (M, K, L) and B (N, K, L) are K-major
with batch outermost, i.e. bytes ordered (L, M, K) / (L, N, K); C is N-major,
(L, M, N).  Arrays here use that (L, rows, K) order.

The oracle is float64.  A decoded element has at most 4 significant bits and
a scale is a power of two, so each product A_hat*B_hat is exact in float64;
only the K-sum rounds (at most K * 2^-53 * sum|A_hat*B_hat|, far below the
comparison tolerance).  The same decoded operands give
S = sum_k |A_hat|*|B_hat|, the per-element scale of the tolerance.

Reading (pages silent): Amax over an empty output (M, N or L zero) is 0, the
identity of a maximum of absolute values; a NaN anywhere in C makes Amax NaN.

Pins (``tests/test_oracle_gemm.py``): exact rational brute force with
``fractions.Fraction`` and torch's float8 decoders on tiny shapes; the
unit-scale special case against torch.matmul on torch-decoded operands; the
identity-operand invariant C = B_hat^T; the scale-doubling invariant (one SFA
byte + 1 changes C by exactly that block's partial sum); sign flip; operand
swap gives C^T; K-block permutation invariance; amax closed form.
"""

import numpy as np

from .codecs import decode, element_codes
from .sf_atom import expand_scales


def _cdiv(a, b):
    return -(-a // b)


def dequantize(codes, fmt, sf_phys, rows, k, l, sf_vec_size):
    """A_hat or B_hat in float64, shape (L, rows, K), from codes (L, rows, K) and the physical SF."""
    codes = element_codes(codes, fmt, rows, k, l)
    scale = expand_scales(sf_phys, rows, k, l, sf_vec_size)          # (L, rows, Kb)
    per_k = np.repeat(scale, sf_vec_size, axis=2)[:, :, :k]           # (L, rows, K)
    return decode(codes, fmt) * per_k


def amax_of(c):
    """max |C| with NaN propagation; 0 for an empty C."""
    c = np.asarray(c)
    if c.size == 0:
        return 0.0
    return float(np.max(np.abs(c)))


def gemm_amax(a, b, sfa, sfb, m, n, k, l, sf_vec_size, a_fmt, b_fmt, want_s=True):
    """Full oracle: returns (C fp64 (L,M,N), S fp64 (L,M,N) or None, Amax float)."""
    ah = dequantize(a, a_fmt, sfa, m, k, l, sf_vec_size)
    bh = dequantize(b, b_fmt, sfb, n, k, l, sf_vec_size)
    with np.errstate(invalid="ignore", over="ignore"):
        c = np.matmul(ah, bh.transpose(0, 2, 1))
        s = np.matmul(np.abs(ah), np.abs(bh).transpose(0, 2, 1)) if want_s else None
    return c, s, amax_of(c)


def gemm_amax_loops(a, b, sfa, sfb, m, n, k, l, sf_vec_size, a_fmt, b_fmt):
    """Plain scalar loops over (l, m, n, k); for tiny shapes only.  Returns (C, S, Amax)."""
    ah = dequantize(a, a_fmt, sfa, m, k, l, sf_vec_size)
    bh = dequantize(b, b_fmt, sfb, n, k, l, sf_vec_size)
    c = np.zeros((l, m, n), dtype=np.float64)
    s = np.zeros((l, m, n), dtype=np.float64)
    for bi in range(l):
        for i in range(m):
            for j in range(n):
                acc = 0.0
                mag = 0.0
                for kk in range(k):
                    p = float(ah[bi, i, kk]) * float(bh[bi, j, kk])
                    acc += p
                    mag += abs(p)
                c[bi, i, j] = acc
                s[bi, i, j] = mag
    return c, s, amax_of(c)


def gemm_rows(a, b, sfa, sfb, m, n, k, l, sf_vec_size, a_fmt, b_fmt, batch, row_idx):
    """C and S for the listed rows of one batch: (len(row_idx), N) each.

    Dequantises only the rows needed from A (all of B for that batch), so it
    can sample outputs of shapes too large for the full oracle.
    """
    row_idx = np.asarray(row_idx, dtype=np.int64)
    a3 = element_codes(a, a_fmt, m, k, l)
    b3 = element_codes(b, b_fmt, n, k, l)
    sa = expand_scales(sfa, m, k, l, sf_vec_size)[batch, row_idx]       # (r, Kb)
    sb = expand_scales(sfb, n, k, l, sf_vec_size)[batch]                # (N, Kb)
    ah = decode(a3[batch, row_idx], a_fmt) * np.repeat(sa, sf_vec_size, axis=1)[:, :k]
    bh = decode(b3[batch], b_fmt) * np.repeat(sb, sf_vec_size, axis=1)[:, :k]
    with np.errstate(invalid="ignore", over="ignore"):
        c = ah @ bh.T
        s = np.abs(ah) @ np.abs(bh).T
    return c, s


def gemm_entries(a, b, sfa, sfb, m, n, k, l, sf_vec_size, a_fmt, b_fmt, idx_l, idx_m, idx_n):
    """C and S at individual output positions (idx_l[i], idx_m[i], idx_n[i])."""
    idx_l = np.asarray(idx_l, dtype=np.int64)
    idx_m = np.asarray(idx_m, dtype=np.int64)
    idx_n = np.asarray(idx_n, dtype=np.int64)
    a3 = element_codes(a, a_fmt, m, k, l)
    b3 = element_codes(b, b_fmt, n, k, l)
    sa_all = expand_scales(sfa, m, k, l, sf_vec_size)
    sb_all = expand_scales(sfb, n, k, l, sf_vec_size)
    ah = decode(a3[idx_l, idx_m], a_fmt) * np.repeat(sa_all[idx_l, idx_m], sf_vec_size, axis=1)[:, :k]
    bh = decode(b3[idx_l, idx_n], b_fmt) * np.repeat(sb_all[idx_l, idx_n], sf_vec_size, axis=1)[:, :k]
    with np.errstate(invalid="ignore", over="ignore"):
        c = np.sum(ah * bh, axis=1)
        s = np.sum(np.abs(ah) * np.abs(bh), axis=1)
    return c, s


def gemm_row_blocks(a, b, sfa, sfb, m, n, k, l, sf_vec_size, a_fmt, b_fmt, block_rows=1024):
    """Every output of the full oracle, one block of rows at a time.

    Yields (batch, first_row, C block, S block), blocks of shape (rows, N) in
    float64, covering all batches and rows in order.  B is dequantised once
    per batch; each block is the same dequantise-and-contract as gemm_amax on
    that slice of A, so the full C and S of shapes too large to hold at once
    can still be checked element by element.
    """
    a3 = element_codes(a, a_fmt, m, k, l)
    b3 = element_codes(b, b_fmt, n, k, l)
    sa = expand_scales(sfa, m, k, l, sf_vec_size)                        # (L, M, Kb)
    sb = expand_scales(sfb, n, k, l, sf_vec_size)                        # (L, N, Kb)
    for batch in range(l):
        bh = decode(b3[batch], b_fmt) * np.repeat(sb[batch], sf_vec_size, axis=1)[:, :k]
        bt, abt = np.ascontiguousarray(bh.T), np.ascontiguousarray(np.abs(bh).T)
        del bh
        for r0 in range(0, m, block_rows):
            r1 = min(m, r0 + block_rows)
            ah = decode(a3[batch, r0:r1], a_fmt) * np.repeat(sa[batch, r0:r1], sf_vec_size, axis=1)[:, :k]
            with np.errstate(invalid="ignore", over="ignore"):
                c = ah @ bt
                s = np.abs(ah) @ abt
            yield batch, r0, c, s

