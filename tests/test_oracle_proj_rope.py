"""Pins of oracle.proj_rope (the projection page's per-head RoPE and dual-direction MXFP8),
checked against what the page and the mathematics fix rather than against its own formulas."""

import numpy as np
import torch

import oracle
from oracle.codecs import decode, FMT_E4M3

H, D, QR = 3, 192, 64
NOPE, R = D - QR, QR // 2


def bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def y_of(t, seed):
    return np.random.default_rng(seed).standard_normal((t, H * D)).astype(np.float32)


def test_identity_angle_is_the_deinterleaving():
    t = 4
    y = y_of(t, 0)
    z = oracle.rope(y, np.ones((t, QR)), np.zeros((t, QR)), H, D, QR)
    y3 = y.reshape(t, H, D)
    assert np.array_equal(z[:, :, :NOPE], y3[:, :, :NOPE])
    assert np.array_equal(z[:, :, NOPE:NOPE + R], y3[:, :, NOPE::2])        # first members, in order
    assert np.array_equal(z[:, :, NOPE + R:], y3[:, :, NOPE + 1::2])       # second members


def test_quarter_turn_sign_convention():
    t = 2
    y = y_of(t, 1)
    z = oracle.rope(y, np.zeros((t, QR)), np.ones((t, QR)), H, D, QR)
    y3 = y.reshape(t, H, D)
    assert np.array_equal(z[:, :, NOPE:NOPE + R], -y3[:, :, NOPE + 1::2])   # -b
    assert np.array_equal(z[:, :, NOPE + R:], y3[:, :, NOPE::2])            # +a


def test_rotation_then_inverse_scales_by_cos2_plus_sin2():
    t = 8
    rng = np.random.default_rng(2)
    theta = rng.uniform(-np.pi, np.pi, size=(t, R))
    c = bf16(np.concatenate([np.cos(theta), np.cos(theta)], axis=1))
    s = bf16(np.concatenate([np.sin(theta), np.sin(theta)], axis=1))
    y = y_of(t, 3)
    z = oracle.rope(y, c, s, H, D, QR)
    # re-interleave the halves and rotate back by the opposite angle
    zi = z.copy()
    zi[:, :, NOPE::2] = z[:, :, NOPE:NOPE + R]
    zi[:, :, NOPE + 1::2] = z[:, :, NOPE + R:]
    back = oracle.rope(zi.reshape(t, H * D), c, -s, H, D, QR).astype(np.float64)
    y3 = y.reshape(t, H, D).astype(np.float64)
    k = (c[:, :R].astype(np.float64) ** 2 + s[:, :R].astype(np.float64) ** 2)[:, None, :]
    want_a, want_b = y3[:, :, NOPE::2] * k, y3[:, :, NOPE + 1::2] * k
    tol = 8 * 2.0 ** -24 * (np.abs(y3[:, :, NOPE::2]) + np.abs(y3[:, :, NOPE + 1::2])) + 1e-30
    assert np.all(np.abs(back[:, :, NOPE:NOPE + R] - want_a) <= tol)
    assert np.all(np.abs(back[:, :, NOPE + R:] - want_b) <= tol)


def _check_direction(vals, codes, scales_per_block, block_axis_len):
    """vals (..., n) float32 in blocks of 32 along the last axis, codes alike, scales (..., n / 32)."""
    v = vals.astype(np.float64).reshape(*vals.shape[:-1], block_axis_len // 32, 32)
    e = scales_per_block.astype(np.int64) - 127
    bm = np.abs(v).max(axis=-1)
    nz = bm > 0
    # minimal exponent: 448 * 2^(e-1) < bm <= 448 * 2^e
    assert np.all(np.ldexp(448.0, e[nz]) >= bm[nz]) and np.all(np.ldexp(448.0, e[nz] - 1) < bm[nz])
    assert np.all(e[~nz] == 0)
    # every code is a nearest E4M3 value of x * 2^-e (brute force over all finite codes)
    q = np.ldexp(v, -e[..., None]).reshape(-1)
    table = decode(np.arange(256, dtype=np.uint8), FMT_E4M3)
    table = table[np.isfinite(table)]
    best = np.min(np.abs(table[None, :] - q[:, None]), axis=1)
    got = decode(codes.reshape(-1), FMT_E4M3)
    assert np.all(np.abs(got - q) == best)


def test_dual_direction_quantisation_definition():
    t = 64
    rng = np.random.default_rng(4)
    y = (rng.standard_normal((t, H * D)) * np.exp2(rng.integers(-6, 7, size=(t, 1)))).astype(np.float32)
    y[5, :D] = 0.0                                        # an all-zero row block
    c = bf16(rng.uniform(-1, 1, size=(t, QR)))
    s = bf16(rng.uniform(-1, 1, size=(t, QR)))
    row, row_s, col, col_s = oracle.proj_rope_mxfp8(y, c, s, H, D, QR)
    assert row.shape == (t, H, D) and row_s.shape == (t, H, D // 32)
    assert col.shape == (t, H, D) and col_s.shape == (t // 32, H, D)
    z = oracle.rope(y, c, s, H, D, QR)
    _check_direction(z, row, row_s, D)
    zt = np.ascontiguousarray(z.transpose(1, 2, 0))       # (H, D, tokens): blocks along tokens
    _check_direction(zt, np.ascontiguousarray(col.transpose(1, 2, 0)),
                     np.ascontiguousarray(col_s.transpose(1, 2, 0)), t)
