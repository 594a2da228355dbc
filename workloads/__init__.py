"""Seeded synthetic inputs for the block-scaled FP8 GEMM + amax.

This module is shared by the tests, the benchmark and the smoke check.  It
draws float32 values, MX-quantises them into 8-bit element codes plus one
E8M0 scale byte per (row, block of ``sf_vec_size`` K elements), and packs
the scale bytes into the physical scale-factor atom buffer.  It performs no
part of the GEMM or the amax, and it imports neither the oracle nor the HIP
library.

MX quantisation recipe (per row and K-block of the float32 input x):

* bm = max |x| over the block;
* e  = the smallest integer with FMAX * 2^e >= bm (FMAX = 448 for E4M3,
  57344 for E5M2), clamped to [-127, 127]; e = 0 when bm = 0;
* scale byte = e + 127;
* code = x * 2^-e, clamped to [-FMAX, FMAX], rounded to the nearest
  representable value with ties to even (torch's float8 cast, which is
  round-to-nearest-even but not saturating -- hence the clamp first).

The SF atom packing follows "GEMM + Amax (SM100)", section "Shapes" (logical
shape) and the physical-shape paragraph of "Using JAX arrays": physical
C-contiguous (L, ceil(MN/128), ceil(K/(4 sf)), 32, 4, 4), where row
mn = i0 + 32*i1 + 128*i2 sits at [.., i2, .., i0, i1, ..] and K-block
kb = i3 + 4*i4 at [.., i4, .., .., .., i3].  Padding entries (rows past MN,
K-blocks past ceil(K/sf)) get ``pad_byte``.

Workloads (seed = workload number, numpy.random.default_rng):

1. tiny        M=N=K=256, L=1, sf=32, E4M3/E4M3, A,B ~ N(0,1)
2. square      M=N=K=2048, L=1, sf=32, E4M3/E4M3, A = sigma*N(0,1) with one
               sigma = 2^U(-8,8) per (row, K-block); B ~ N(0,1)
3. batched     L=8, M=N=K=4096, sf=32, E4M3/E4M3, N(0,1); A[l*,m*,k*] = +1e4
4. ragged      M=4000, N=7168, K=2048, L=1, sf=16, A E5M2, B E4M3,
               Student-t(3) values
5. projection  M=8192, N=24576 (128 heads x 192), K=1536, L=1, sf=32,
               E4M3/E4M3, A ~ N(0,1), B ~ N(0,1)/sqrt(K)
"""

import math

import numpy as np

FMT_E4M3 = 0
FMT_E5M2 = 1
FMT_E2M1 = 2     # packed FP4: two elements per byte, element 2i in the low nibble
FMAX = {FMT_E4M3: 448.0, FMT_E5M2: 57344.0, FMT_E2M1: 6.0}

WORKLOADS = {
    1: dict(name="tiny", M=256, N=256, K=256, L=1, sf=32, a_fmt=FMT_E4M3, b_fmt=FMT_E4M3),
    2: dict(name="square", M=2048, N=2048, K=2048, L=1, sf=32, a_fmt=FMT_E4M3, b_fmt=FMT_E4M3),
    3: dict(name="batched", M=4096, N=4096, K=4096, L=8, sf=32, a_fmt=FMT_E4M3, b_fmt=FMT_E4M3),
    4: dict(name="ragged", M=4000, N=7168, K=2048, L=1, sf=16, a_fmt=FMT_E5M2, b_fmt=FMT_E4M3),
    5: dict(name="projection", M=8192, N=24576, K=1536, L=1, sf=32, a_fmt=FMT_E4M3, b_fmt=FMT_E4M3),
}


def cdiv(a, b):
    return -(-a // b)


def sf_bytes(mn, k, l, sf_vec_size):
    """Size in bytes of the physical SF buffer."""
    return 512 * l * cdiv(mn, 128) * cdiv(k, 4 * sf_vec_size)


def _torch_fp8(fmt):
    import torch
    return torch.float8_e4m3fn if fmt == FMT_E4M3 else torch.float8_e5m2


def block_exponents(x, sf_vec_size, fmt):
    """Per-block exponent e (int32, shape (L, rows, Kb)) of the MX recipe for float32 x (L, rows, K)."""
    l, rows, k = x.shape
    kb = cdiv(k, sf_vec_size)
    pad = kb * sf_vec_size - k
    ax = np.abs(x)
    if pad:
        ax = np.concatenate([ax, np.zeros((l, rows, pad), dtype=ax.dtype)], axis=2)
    bm = ax.reshape(l, rows, kb, sf_vec_size).max(axis=3).astype(np.float64)
    fmax = FMAX[fmt]
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(bm / fmax))
    e = np.where(bm > 0, e, 0.0)
    e = np.clip(e, -300, 300)
    # exact correction of log2 rounding: smallest e with fmax*2^e >= bm
    e = np.where((bm > 0) & (np.ldexp(fmax, (e - 1).astype(np.int64)) >= bm), e - 1, e)
    e = np.where((bm > 0) & (np.ldexp(fmax, e.astype(np.int64)) < bm), e + 1, e)
    e = np.clip(e, -127, 127)
    return e.astype(np.int32)


def _e2m1_rne(q):
    """Nearest E2M1 value code (4-bit, sign in bit 3) of float64 q with |q| <= 6, ties to even.

    The E2M1 grid is spaced 0.5 on [0, 2), 1 on [2, 4) and 2 on [4, 6]; numpy's round is
    half-to-even, and the even multiple is always the code with the even mantissa."""
    a = np.abs(q)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    v = np.round(a / step) * step
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    code = np.searchsorted(grid, v).astype(np.uint8)
    assert np.array_equal(grid[code], v)
    return np.where(np.signbit(q), code | 0x8, code).astype(np.uint8)


def mx_quantize(x, sf_vec_size, fmt):
    """MX-quantise float32 x (L, rows, K): returns (codes uint8 (L,rows,K), scale bytes uint8 (L,rows,Kb)).

    E2M1 codes come packed, (L, rows, K/2) bytes."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    l, rows, k = x.shape
    e = block_exponents(x, sf_vec_size, fmt)
    per_k = np.repeat(e, sf_vec_size, axis=2)[:, :, :k].astype(np.int64)
    q = np.ldexp(x.astype(np.float64), -per_k)
    fmax = FMAX[fmt]
    q = np.clip(q, -fmax, fmax).astype(np.float32)
    if fmt == FMT_E2M1:
        assert k % 2 == 0, "packed FP4 rows need an even K"
        n = _e2m1_rne(q.astype(np.float64))
        return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8), (e + 127).astype(np.uint8)
    codes = torch.from_numpy(q).to(_torch_fp8(fmt)).view(torch.uint8).numpy()
    return codes, (e + 127).astype(np.uint8)


def pack_sf(scale_bytes, mn, k, l, sf_vec_size, pad_byte=127):
    """Pack per-(batch, row, K-block) scale bytes (L, MN, Kb) into the flat physical SF buffer."""
    mnb = cdiv(mn, 128)
    kg = cdiv(k, 4 * sf_vec_size)
    kb = cdiv(k, sf_vec_size)
    full = np.full((l, mnb * 128, kg * 4), pad_byte, dtype=np.uint8)
    full[:, :mn, :kb] = np.asarray(scale_bytes, dtype=np.uint8).reshape(l, mn, kb)
    # axes (l, i2, i1, i0, i4, i3) -> physical (l, i2, i4, i0, i1, i3)
    phys = full.reshape(l, mnb, 4, 32, kg, 4).transpose(0, 1, 4, 3, 2, 5)
    return np.ascontiguousarray(phys).reshape(-1)


def _draw_normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def make_problem(M, N, K, L, sf, a_fmt, b_fmt, seed, dist="normal", pad_byte=127,
                 a_sigma_blocks=False, b_scale=1.0, outlier=None):
    """Quantised inputs for one problem.

    Returns a dict with A (L,M,K) uint8, B (L,N,K) uint8, SFA / SFB flat
    physical uint8 buffers, and the shape/format fields.
    """
    rng = np.random.default_rng(seed)
    sigma = None
    if a_sigma_blocks:
        kb = cdiv(K, sf)
        sigma = np.exp2(rng.uniform(-8.0, 8.0, size=(L, M, kb))).astype(np.float32)
    if dist == "normal":
        xa = _draw_normal(rng, (L, M, K))
        xb = _draw_normal(rng, (L, N, K))
    elif dist == "student_t3":
        xa = rng.standard_t(3, size=(L, M, K)).astype(np.float32)
        xb = rng.standard_t(3, size=(L, N, K)).astype(np.float32)
    elif dist == "uniform_codes":
        xa = rng.uniform(-4.0, 4.0, size=(L, M, K)).astype(np.float32)
        xb = rng.uniform(-4.0, 4.0, size=(L, N, K)).astype(np.float32)
    else:
        raise ValueError(dist)
    if sigma is not None:
        xa *= np.repeat(sigma, sf, axis=2)[:, :, :K]
    if b_scale != 1.0:
        xb *= np.float32(b_scale)
    out_pos = None
    if outlier is not None:
        ol = int(rng.integers(0, L))
        om = int(rng.integers(0, M))
        ok = int(rng.integers(0, K))
        xa[ol, om, ok] = np.float32(outlier)
        out_pos = (ol, om, ok)
    a_codes, a_sb = mx_quantize(xa, sf, a_fmt)
    del xa
    b_codes, b_sb = mx_quantize(xb, sf, b_fmt)
    del xb
    return dict(
        A=a_codes, B=b_codes,
        SFA=pack_sf(a_sb, M, K, L, sf, pad_byte), SFB=pack_sf(b_sb, N, K, L, sf, pad_byte),
        M=M, N=N, K=K, L=L, sf=sf, a_fmt=a_fmt, b_fmt=b_fmt, outlier=out_pos,
    )


def make_workload(i, seed=None, pad_byte=127):
    """Inputs of workload i (1..5), seeded with ``seed`` (default: i)."""
    w = WORKLOADS[i]
    seed = i if seed is None else seed
    kw = dict(M=w["M"], N=w["N"], K=w["K"], L=w["L"], sf=w["sf"], a_fmt=w["a_fmt"],
              b_fmt=w["b_fmt"], seed=seed, pad_byte=pad_byte)
    if i == 2:
        return make_problem(a_sigma_blocks=True, **kw)
    if i == 3:
        return make_problem(outlier=1.0e4, **kw)
    if i == 4:
        return make_problem(dist="student_t3", **kw)
    if i == 5:
        return make_problem(b_scale=1.0 / math.sqrt(w["K"]), **kw)
    return make_problem(**kw)


def flops(M, N, K, L):
    """Algorithmic flop count 2*M*N*K*L of one GEMM."""
    return 2 * M * N * K * L


def algorithmic_bytes(M, N, K, L, sf):
    """A + B + SFA + SFB read once, fp32 C written once, plus the 4-byte Amax."""
    return M * K * L + N * K * L + sf_bytes(M, K, L, sf) + sf_bytes(N, K, L, sf) + 4 * M * N * L + 4
