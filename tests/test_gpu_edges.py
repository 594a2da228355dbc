"""GPU parity at the edges of the value range, through the C ABI.

* Scale bytes at both ends of the range where the default datapath dequantises
  every code exactly (bf16 holds every code times 2^(byte-127)): 3 and 246 for
  E4M3, 10 and 239 for E5M2, with every finite code, subnormals and the
  largest included.  The bytes alternate per K-block between the two
  operands so that every product stays inside float32's range.
* One byte beyond each end, codes whose dequantised value is still a bf16
  number (the claim is that these stay exact too).
* NaN and infinity element codes (E4M3 0x7F / 0xFF, E5M2 0x7C / 0xFC and
  0x7D): the NaN and infinity pattern of C and the NaN Amax must be the
  oracle's (IEEE float64 arithmetic on the decoded values).
* Same-sign data with long K, where the float32 accumulation error is
  largest: the error must stay within the bound the header states as a
  function of K, and within the contract bound up to K = 2048.
* Amax across workgroups: every workgroup issues at most one atomic and skips
  it when Amax already holds its maximum.  With every output equal, and with
  one outlier row in the first, a middle or the last tile (one-round and
  multi-round grids), Amax must be the closed-form maximum.
"""

import numpy as np
import pytest

import oracle
import workloads as W
from parity_util import amax_bits_of, check_amax, check_c, fetch, float_bits, run, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

E4, E5 = W.FMT_E4M3, W.FMT_E5M2
TILES = {"t128": 4, "t256": 8}
# scale bytes at the ends of the exact range, per format
EXACT_RANGE = {E4: (3, 246), E5: (10, 239)}


@pytest.fixture(scope="module")
def lib():
    import block_scaled_precision_e4m3_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return lib


def finite_codes(fmt):
    b = np.arange(256, dtype=np.uint8)
    if fmt == E4:
        return b[(b & 0x7F) != 0x7F]
    return b[((b >> 2) & 0x1F) != 0x1F]


def problem(a, b, sa, sb, sf, fa, fb):
    """A problem dict from explicit codes (L, rows, K) and scale bytes (L, rows, Kb)."""
    L, M, K = a.shape
    N = b.shape[1]
    return dict(A=np.ascontiguousarray(a), B=np.ascontiguousarray(b), SFA=W.pack_sf(sa, M, K, L, sf),
                SFB=W.pack_sf(sb, N, K, L, sf), M=M, N=N, K=K, L=L, sf=sf, a_fmt=fa, b_fmt=fb, outlier=None)


def oracle_full(p):
    return oracle.gemm_amax(p["A"], p["B"], p["SFA"], p["SFB"], p["M"], p["N"], p["K"], p["L"], p["sf"],
                            p["a_fmt"], p["b_fmt"])


def run_fetch(lib, p, tile):
    d = to_device(p)
    run(lib, p, d, flags=TILES[tile])
    return fetch(p, d)


def alternating_bytes(L, rows, kb, first, second):
    """Scale bytes that are `first` on even K-blocks and `second` on odd ones."""
    row = np.where(np.arange(kb) % 2 == 0, first, second).astype(np.uint8)
    return np.broadcast_to(row, (L, rows, kb)).copy()


@pytest.mark.parametrize("tile", list(TILES))
@pytest.mark.parametrize("sf", [32, 16])
@pytest.mark.parametrize("fa,fb", [(E4, E4), (E5, E4), (E4, E5), (E5, E5)])
def test_scale_bytes_at_the_ends_of_the_exact_range(lib, fa, fb, sf, tile):
    M, N, K, L = 300, 260, 512, 1
    rng = np.random.default_rng(31 + 4 * fa + fb)
    a = rng.choice(finite_codes(fa), size=(L, M, K)).astype(np.uint8)
    b = rng.choice(finite_codes(fb), size=(L, N, K)).astype(np.uint8)
    # every row also holds the smallest subnormal and the largest code
    a[:, :, 0], a[:, :, 1] = 0x01, (0x7E if fa == E4 else 0x7B)
    b[:, :, 0], b[:, :, 1] = (0x7E if fb == E4 else 0x7B), 0x01
    a[:, :, sf], b[:, :, sf] = 0x81, 0x01
    (alo, ahi), (blo, bhi) = EXACT_RANGE[fa], EXACT_RANGE[fb]
    kb = -(-K // sf)
    p = problem(a, b, alternating_bytes(L, M, kb, ahi, alo), alternating_bytes(L, N, kb, blo, bhi), sf, fa, fb)
    c, amax = run_fetch(lib, p, tile)
    c_ref, s_ref, amax_ref = oracle_full(p)
    assert np.all(np.isfinite(c_ref))
    ratio = check_c(c, c_ref, s_ref, f"scale bytes {alo}/{ahi} x {blo}/{bhi}")
    check_amax(amax, amax_ref)
    assert float_bits(amax) == amax_bits_of(c)
    print(f"  max |diff|/bound = {ratio:.3g}", flush=True)


def bf16_representable(values):
    """True where a float64 value is exactly a finite bfloat16 number (subnormals included)."""
    v = np.asarray(values, dtype=np.float64)
    t = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    return np.isfinite(t) & (t == v)


@pytest.mark.parametrize("tile", list(TILES))
@pytest.mark.parametrize("fmt", [E4, E5])
def test_scale_bytes_beyond_the_range_with_representable_codes(lib, fmt, tile):
    # One byte past each end: only codes whose dequantised value fits bf16 are
    # used, and those must stay exact.
    M, N, K, L, sf = 160, 132, 256, 1, 32
    lo, hi = EXACT_RANGE[fmt]
    codes = finite_codes(fmt)
    vals = oracle.decode(codes, fmt)
    ok_lo = codes[bf16_representable(vals * 2.0 ** (lo - 1 - 127))]
    ok_hi = codes[bf16_representable(vals * 2.0 ** (hi + 1 - 127))]
    assert 0 < len(ok_lo) < len(codes) and 0 < len(ok_hi) < len(codes)
    rng = np.random.default_rng(41 + fmt)
    kb = K // sf
    a = np.empty((L, M, K), dtype=np.uint8)
    for j in range(kb):
        pool = ok_hi if j % 2 == 0 else ok_lo
        a[:, :, j * sf:(j + 1) * sf] = rng.choice(pool, size=(L, M, sf))
    b = rng.choice(finite_codes(E4), size=(L, N, K)).astype(np.uint8)
    # B's bytes bring each product back into float32's range
    sa = alternating_bytes(L, M, kb, hi + 1, lo - 1)
    sb = alternating_bytes(L, N, kb, 254 - (hi + 1), 254 - (lo - 1) - 100)
    p = problem(a, b, sa, sb, sf, fmt, E4)
    c, amax = run_fetch(lib, p, tile)
    c_ref, s_ref, amax_ref = oracle_full(p)
    assert np.all(np.isfinite(c_ref))
    ratio = check_c(c, c_ref, s_ref, f"bytes {lo - 1}/{hi + 1}")
    check_amax(amax, amax_ref)
    print(f"  max |diff|/bound = {ratio:.3g}", flush=True)


@pytest.mark.parametrize("tile", list(TILES))
@pytest.mark.parametrize("fa,fb", [(E4, E5), (E5, E5)])
def test_nan_and_inf_element_codes(lib, fa, fb, tile):
    M, N, K, L, sf = 200, 136, 256, 2, 32
    p = W.make_problem(M, N, K, L, sf, fa, fb, seed=51 + fa)
    a, b = p["A"].copy(), p["B"].copy()
    a_nan = 0x7F if fa == E4 else 0x7D
    a[1, 5, 17] = a_nan                  # NaN: row 5 of batch 1 all NaN
    a[0, 150, 200] = a_nan | 0x80        # negative NaN code
    b[0, 9, 40] = 0x7C                   # +inf and -inf in one B row: inf - inf or +-inf per A
    b[0, 9, 41] = 0xFC
    b[1, 20, 3] = 0x7C                   # +inf alone: +-inf, NaN where A's code is zero
    a[1, 7, 3] = 0x00
    b[0, 130, 64] = 0xFC
    if fa == E5:
        a[0, 60, 100] = 0xFC             # -inf in A
    p["A"], p["B"] = a, b
    c, amax = run_fetch(lib, p, tile)
    c_ref, s_ref, _ = oracle_full(p)
    nan_ref, inf_ref = np.isnan(c_ref), np.isinf(c_ref)
    assert nan_ref.any() and inf_ref.any()
    assert np.array_equal(np.isnan(c), nan_ref), f"NaN pattern differs at {np.argwhere(np.isnan(c) != nan_ref)[:5]}"
    assert np.array_equal(np.isinf(c), inf_ref), f"inf pattern differs at {np.argwhere(np.isinf(c) != inf_ref)[:5]}"
    assert np.array_equal(np.sign(c[inf_ref]), np.sign(c_ref[inf_ref]))
    fin = np.isfinite(c_ref)
    check_c(c[fin], c_ref[fin], s_ref[fin], "finite outputs")
    assert np.isnan(amax)


@pytest.mark.parametrize("tile", list(TILES))
@pytest.mark.parametrize("K", [2048, 4096, 16384, 65536])
def test_same_sign_long_k(lib, K, tile):
    # Every product positive: the float32 accumulation error grows with K
    # without cancelling.  Bound stated in the header: (K/16 + 1) * 2^-24 * S;
    # within the contract bound 1e-5 * S for K <= 2048.
    M, N, L, sf = 64, 96, 1, 32
    rng = np.random.default_rng(61)
    pos = finite_codes(E4)
    pos = pos[(pos < 0x80) & (pos >= 0x30) & (pos <= 0x4F)]   # +0.5 .. +3.75
    a = rng.choice(pos, size=(L, M, K)).astype(np.uint8)
    b = rng.choice(pos, size=(L, N, K)).astype(np.uint8)
    kb = K // sf
    p = problem(a, b, np.full((L, M, kb), 127, np.uint8), np.full((L, N, kb), 127, np.uint8), sf, E4, E4)
    c, amax = run_fetch(lib, p, tile)
    c_ref, s_ref, amax_ref = oracle_full(p)
    rel = np.abs(c.astype(np.float64) - c_ref) / s_ref
    model = (K / 16 + 1) * 2.0 ** -24
    print(f"  K={K}: max |diff|/S = {rel.max():.3g} = {rel.max() / 1e-5:.3g} x 1e-5, model bound {model:.3g}",
          flush=True)
    assert rel.max() <= model
    if K <= 2048:
        check_c(c, c_ref, s_ref, f"same sign K={K}")
        check_amax(amax, amax_ref)


@pytest.mark.parametrize("tile", list(TILES))
@pytest.mark.parametrize("M,N", [(1024, 1024), (4096, 2304)])
@pytest.mark.parametrize("where", ["none", "first", "middle", "last"])
def test_amax_across_workgroups(lib, M, N, where, tile):
    # Codes 1.0 (0x38) everywhere and scale bytes 127: every output is exactly K.
    # An outlier row gets scale bytes 131 on A, so that row is exactly 16 K.
    # 1024 x 1024 is one round of tiles; 4096 x 2304 at 128 x 128 tiles is 576
    # tiles in three rounds (at 256 x 256, 144 tiles in one).
    K, L, sf, fmt = 128, 1, 32, E4
    kb = K // sf
    a = np.full((L, M, K), 0x38, dtype=np.uint8)
    b = np.full((L, N, K), 0x38, dtype=np.uint8)
    sa = np.full((L, M, kb), 127, dtype=np.uint8)
    sb = np.full((L, N, kb), 127, dtype=np.uint8)
    row = {"none": None, "first": 0, "middle": M // 2 + 37, "last": M - 1}[where]
    if row is not None:
        sa[:, row, :] = 131
    p = problem(a, b, sa, sb, sf, fmt, fmt)
    c, amax = run_fetch(lib, p, tile)
    expect = np.full((L, M, N), float(K), dtype=np.float32)
    if row is not None:
        expect[:, row, :] = 16.0 * K
    assert np.array_equal(c, expect), f"C differs from the closed form ({where} outlier)"
    assert float_bits(amax) == float_bits(16.0 * K if row is not None else float(K)), \
        f"Amax {amax} ({where} outlier, {M}x{N}, {tile})"
