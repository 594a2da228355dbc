"""Per-head RoPE and dual-direction MXFP8 quantisation of a projection output.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes ("GEMM + RoPE + MXFP8 Projection (SM100)", sections
"Overview", "Shapes" and "Equations"): the projection Y (tokens, NUM_HEADS *
HEAD_DIM) viewed as (tokens, NUM_HEADS, HEAD_DIM); RoPE applied to the
trailing QK_ROPE features of every head (the leading QK_NOPE features pass
through); then MXFP8 (E4M3 codes, E8M0 scale per block of 32) twice: blocks
along HEAD_DIM ("row", D-direction) and blocks along tokens ("col",
S-direction).

Readings of what the page leaves open:

* RoPE, "interleaved-in / halves-out": the QK_ROPE inputs of a head are
  pairs (a_i, b_i) = (y[2i], y[2i+1]), i < R = QK_ROPE / 2; the output holds
  the rotated first members in positions i and the second members in
  positions R + i:
      out[i]     = a_i * cos[i]     - b_i * sin[i]
      out[R + i] = b_i * cos[R + i] + a_i * sin[R + i]
  with cos / sin the token's QK_ROPE-entry bf16 rows (the usual rotate-half
  form applied after de-interleaving).  Arithmetic in float32, each product
  and the sum rounded separately (no fused multiply-add), so that the GPU,
  doing the same, reaches bitwise the same values and hence the same codes.
* MXFP8 scale rule: the one the GEMM's own inputs use (``mx_quantize``):
  e = the smallest integer with 448 * 2^e >= max |block|, clamped to
  [-127, 127], 0 for an all-zero block; codes round x * 2^-e to nearest,
  ties to even.
* Layouts (page section "Shapes"): codes (tokens, H, D) in both directions;
  row scales (tokens, H, D / 32); column scales (tokens / 32, H, D).

Pins (``tests/test_oracle_proj_rope.py``): cos = 1, sin = 0 reduces RoPE to
the de-interleaving permutation; cos = 0, sin = 1 gives (-b, a); each output
pair is the plane rotation of its input pair (norm kept in float64, and the
float32 result within rounding of the exact rotation); the QK_NOPE features
pass unchanged; both directions' scale exponents are minimal for their own
blocks and every code is the nearest to its value (checked against the
float64 block maxima and a brute-force search, not through ``mx_quantize``).
"""

import numpy as np

from .codecs import FMT_E4M3
from .mx_quantize import block_exponent, encode_rne


def rope(y, cos, sin, num_heads, head_dim, qk_rope):
    """float32 (tokens, num_heads * head_dim) -> float32 (tokens, num_heads, head_dim) with RoPE on the tail."""
    y = np.asarray(y, dtype=np.float32)
    t = y.shape[0]
    y = y.reshape(t, num_heads, head_dim).copy()
    r = qk_rope // 2
    nope = head_dim - qk_rope
    c = np.asarray(cos, dtype=np.float32)[:, None, :]   # (tokens, 1, qk_rope)
    s = np.asarray(sin, dtype=np.float32)[:, None, :]
    a = y[:, :, nope + 0:head_dim:2]                     # (tokens, H, r): y[2i]
    b = y[:, :, nope + 1:head_dim:2]                     # y[2i+1]
    first = np.subtract(np.multiply(a, c[:, :, :r], dtype=np.float32),
                        np.multiply(b, s[:, :, :r], dtype=np.float32), dtype=np.float32)
    second = np.add(np.multiply(b, c[:, :, r:], dtype=np.float32),
                    np.multiply(a, s[:, :, r:], dtype=np.float32), dtype=np.float32)
    out = y.copy()
    out[:, :, nope:nope + r] = first
    out[:, :, nope + r:] = second
    return out


def _quantize_blocks(v, block):
    """float32 (..., n) with n % block == 0 -> (codes uint8 (..., n), scale bytes (..., n / block)), E4M3."""
    v = np.asarray(v, dtype=np.float32)
    shp = v.shape
    n = shp[-1]
    blocks = v.astype(np.float64).reshape(*shp[:-1], n // block, block)
    bm = np.abs(blocks).max(axis=-1)
    e = block_exponent(bm, FMT_E4M3)
    q = np.ldexp(blocks, -e[..., None])
    codes = encode_rne(q, FMT_E4M3).reshape(shp)
    return codes, (e + 127).astype(np.uint8)


def proj_rope_mxfp8(y, cos, sin, num_heads, head_dim, qk_rope, block=32):
    """Y (tokens, H*D) float32 -> (out_fp8_row, out_scales_row, out_fp8_col, out_scales_col)."""
    z = rope(y, cos, sin, num_heads, head_dim, qk_rope)              # (tokens, H, D)
    t = z.shape[0]
    assert head_dim % block == 0 and t % block == 0
    row_codes, row_scales = _quantize_blocks(z, block)               # blocks along D
    zc = np.ascontiguousarray(z.transpose(1, 2, 0))                  # (H, D, tokens)
    col_codes_t, col_scales_t = _quantize_blocks(zc, block)          # blocks along tokens
    col_codes = np.ascontiguousarray(col_codes_t.transpose(2, 0, 1))  # (tokens, H, D)
    col_scales = np.ascontiguousarray(col_scales_t.transpose(2, 0, 1))  # (tokens / 32, H, D)
    return row_codes, row_scales, col_codes, col_scales
