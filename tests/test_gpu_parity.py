"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Small shapes (several tiles, ragged M/N, K tails, both sf_vec_size values,
all format pairs, both tile configurations) are compared element by element
with the full fp64 oracle.  The five workloads run at their full sizes in the
launch configuration the benchmark times, every output against the oracle
(computed in row blocks), Amax against the oracle's, plus properties that
hold at any size (Amax equals max |C_gpu| bitwise; every output written).
"""

import numpy as np
import pytest

import oracle
import workloads as W
from parity_util import (amax_bits_of, check_amax, check_c, fetch, float_bits, run, to_device)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

E4, E5 = W.FMT_E4M3, W.FMT_E5M2

# tile configuration flags of mxgemm_amax_ex (0 = the library's own choice)
TILES = {"auto": 0, "t128": 4, "t256": 8}


@pytest.fixture(scope="module")
def lib():
    import block_scaled_precision_e4m3_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert (lib.MXG_FLAG_TILE_128, lib.MXG_FLAG_TILE_256) == (TILES["t128"], TILES["t256"])
    return lib


def _oracle_full(p):
    return oracle.gemm_amax(p["A"], p["B"], p["SFA"], p["SFB"], p["M"], p["N"], p["K"], p["L"], p["sf"],
                            p["a_fmt"], p["b_fmt"])


SMALL = [
    # M, N, K, L, sf, fa, fb
    (300, 520, 592, 2, 32, E4, E4),     # ragged M/N, K % 128 = 80, partial last sf block
    (257, 260, 336, 1, 16, E5, E4),     # sf=16, K % 64 = 16
    (128, 128, 128, 1, 32, E5, E5),
    (1000, 772, 1040, 1, 16, E4, E5),
    (64, 36, 48, 3, 32, E4, E4),        # one partial tile per batch, K < 2 blocks
    (33, 4, 16, 1, 16, E5, E5),         # minimal K and N
    (4096, 4096, 272, 1, 32, E4, E4),   # large enough for the 256x256 tile path
    (4000, 4100, 208, 1, 16, E5, E4),   # 256x256 path, ragged, sf=16
]


@pytest.mark.parametrize("tile", list(TILES))
@pytest.mark.parametrize("dist", ["normal", "student_t3"])
@pytest.mark.parametrize("M,N,K,L,sf,fa,fb", SMALL)
def test_small_shapes_full_oracle(lib, M, N, K, L, sf, fa, fb, dist, tile):
    print(f"case M={M} N={N} K={K} L={L} sf={sf} fmt={fa}{fb} {dist} tile={tile} "
          f"auto={lib.mxgemm_launch_config(M, N, K, L, sf)}", flush=True)
    p = W.make_problem(M, N, K, L, sf, fa, fb, seed=M + N + K, dist=dist)
    d = to_device(p)
    run(lib, p, d, flags=TILES[tile])
    c, amax = fetch(p, d)
    c_ref, s_ref, amax_ref = _oracle_full(p)
    ratio = check_c(c, c_ref, s_ref, f"{M}x{N}x{K}x{L}")
    check_amax(amax, amax_ref)
    assert float_bits(amax) == amax_bits_of(c)
    print(f"  max |diff|/bound = {ratio:.3g}", flush=True)


# The opt-in FP8 matrix path keeps, per 8-element K group, only the bits of
# each product down to 2^-13 of the group's largest product P, so at most 7
# products lose less than 2^-13 * P <= 2^-13 * sum|p| each: |error| stays
# below 2^-10 * sum_k |A_hat||B_hat| (plus fp32 rounding).
FP8_MFMA_REL = 2.0 ** -10


@pytest.mark.parametrize("tile", ["t128", "t256"])
@pytest.mark.parametrize("dist", ["normal", "student_t3"])
@pytest.mark.parametrize("M,N,K,L,sf,fa,fb", SMALL[:6])
def test_fp8_mfma_mode_within_model_bound(lib, M, N, K, L, sf, fa, fb, dist, tile):
    print(f"fp8-mfma case M={M} N={N} K={K} L={L} sf={sf} fmt={fa}{fb} {dist} tile={tile}", flush=True)
    p = W.make_problem(M, N, K, L, sf, fa, fb, seed=M + N + K, dist=dist)
    d = to_device(p)
    run(lib, p, d, flags=lib.MXG_FLAG_FP8_MFMA | TILES[tile])
    c, amax = fetch(p, d)
    c_ref, s_ref, amax_ref = _oracle_full(p)
    err = np.abs(c.astype(np.float64) - c_ref)
    bound = FP8_MFMA_REL * s_ref + 1e-30
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"
    assert float_bits(amax) == amax_bits_of(c)
    print(f"  max |diff|/(1e-5 S) = {np.max(err / (1e-5 * s_ref + 1e-30)):.3g}", flush=True)


# Workloads whose data make the FP8 datapath miss the contract bound: widely
# varying scales within a K-block pair (workload 2) and heavy tails (workload 4)
# put products far below their 8-element group's largest, which that
# datapath truncates.
FP8_MISSES = (2, 4)


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_workload_full_oracle(lib, wid):
    # The workload at full size, in the launch configuration the benchmark
    # times, against the fp64 oracle over every output (row blocks of 1024),
    # including the ragged last tile of workload 4 and the planted outlier of
    # workload 3, whose row holds Amax.  The same inputs also go through the
    # opt-in FP8 datapath, whose largest error relative to the contract bound
    # 1e-5 * S is reported and, where it misses, asserted to miss.
    w = W.WORKLOADS[wid]
    print(f"workload {wid} config={lib.mxgemm_launch_config(w['M'], w['N'], w['K'], w['L'], w['sf'])}", flush=True)
    p = W.make_workload(wid)
    d = to_device(p)
    run(lib, p, d)
    c, amax = fetch(p, d)
    assert float_bits(amax) == amax_bits_of(c)
    run(lib, p, d, flags=lib.MXG_FLAG_FP8_MFMA)
    c8, amax8 = fetch(p, d)
    assert float_bits(amax8) == amax_bits_of(c8)
    args = (p["A"], p["B"], p["SFA"], p["SFB"], p["M"], p["N"], p["K"], p["L"], p["sf"], p["a_fmt"], p["b_fmt"])
    worst = worst8 = amax_ref = 0.0
    for batch, r0, cb, sb in oracle.gemm_row_blocks(*args, block_rows=1024):
        rows = slice(r0, r0 + cb.shape[0])
        worst = max(worst, check_c(c[batch, rows], cb, sb, f"workload {wid} batch {batch} rows {r0}.."))
        worst8 = max(worst8, float(np.max(np.abs(c8[batch, rows] - cb) / (1e-5 * sb + 1e-30))))
        amax_ref = max(amax_ref, oracle.amax_of(cb))
    check_amax(amax, amax_ref, f"workload {wid}")
    if p["outlier"]:
        ol, om, _ = p["outlier"]
        cr, _ = oracle.gemm_rows(*args, ol, [om])
        assert abs(oracle.amax_of(cr) - amax_ref) <= 1e-12 * amax_ref, "the outlier's row holds the largest |C|"
    print(f"  default datapath: max |diff|/bound {worst:.3g}, amax rel err {abs(amax - amax_ref) / amax_ref:.3g}; "
          f"FP8 datapath: max |diff|/(1e-5 S) {worst8:.3g}, amax rel err {abs(amax8 - amax_ref) / amax_ref:.3g}",
          flush=True)
    if wid in FP8_MISSES:
        assert worst8 > 1.0, "the FP8 datapath was expected to miss the contract bound here"


@pytest.mark.parametrize("tile", ["t128", "t256"])
def test_scale_plus_one_doubles_bitwise(lib, tile):
    p = W.make_problem(520, 264, 384, 2, 32, E4, E5, seed=11)
    d = to_device(p)
    run(lib, p, d, flags=TILES[tile])
    c0, a0 = fetch(p, d)
    d["SFA"] += 1          # every scale byte +1: 2x every product (bytes stay < 255 here)
    run(lib, p, d, flags=TILES[tile])
    c1, a1 = fetch(p, d)
    assert np.array_equal(c1, 2 * c0)
    assert a1 == 2 * a0


@pytest.mark.parametrize("tile", ["t128", "t256"])
def test_sign_flip_negates(lib, tile):
    # Flipping every A sign bit negates C.  The bf16 MFMA truncates its
    # 16-product partial sums toward zero before the round-to-nearest add into
    # the accumulator, so the negation is checked to the tolerance rather than
    # bitwise; the count of bitwise differences is reported.
    p = W.make_problem(300, 200, 256, 1, 16, E5, E4, seed=12)
    d = to_device(p)
    run(lib, p, d, flags=TILES[tile])
    c0, a0 = fetch(p, d)
    d["A"] ^= 0x80
    run(lib, p, d, flags=TILES[tile])
    c1, a1 = fetch(p, d)
    _, s_ref, _ = _oracle_full(p)
    assert np.all(np.abs(c1.astype(np.float64) + c0) <= 2e-5 * s_ref)
    assert abs(a1 - a0) <= 1e-5 * a0
    print(f"  bitwise-different entries: {int(np.sum(c1 != -c0))} of {c0.size}", flush=True)


@pytest.mark.parametrize("tile", ["t128", "t256"])
def test_deterministic_and_padding_poison(lib, tile):
    # padding SF bytes set to 0xFF (NaN scale) must never reach the result
    p = W.make_problem(200, 196, 592, 2, 32, E4, E4, seed=13, pad_byte=0xFF)
    d = to_device(p)
    run(lib, p, d, flags=TILES[tile])
    c0, a0 = fetch(p, d)
    run(lib, p, d, flags=TILES[tile])
    c1, a1 = fetch(p, d)
    assert np.array_equal(c0.view(np.uint32), c1.view(np.uint32)) and a0 == a1
    c_ref, s_ref, amax_ref = _oracle_full(p)
    check_c(c0, c_ref, s_ref, "poisoned padding")
    check_amax(a0, amax_ref)


@pytest.mark.parametrize("tile", ["t128", "t256"])
def test_guard_band_untouched(lib, tile):
    p = W.make_problem(130, 68, 160, 2, 16, E4, E4, seed=14)
    pad = 1024
    d = to_device(p, pad_c=pad, c_fill=12345.0)
    run(lib, p, d, flags=TILES[tile])
    torch.cuda.synchronize()
    full = d["C_full"].cpu().numpy()
    assert np.all(full[:pad] == 12345.0) and np.all(full[-pad:] == 12345.0)
    assert not np.any(full[pad:-pad] == 12345.0)


def test_accumulate_flag(lib):
    p = W.make_problem(128, 128, 128, 1, 32, E4, E4, seed=15)
    d = to_device(p)
    run(lib, p, d)
    c, amax = fetch(p, d)
    d["Amax"].fill_(1e30)
    run(lib, p, d, flags=lib.MXG_FLAG_AMAX_ACCUMULATE)
    assert fetch(p, d)[1] == np.float32(1e30)
    d["Amax"].fill_(0.0)
    run(lib, p, d, flags=lib.MXG_FLAG_AMAX_ACCUMULATE)
    assert fetch(p, d)[1] == amax
    lib.mxgemm_amax_reset(d["Amax"])
    assert fetch(p, d)[1] == 0.0


def test_empty_and_k_zero(lib):
    dev = torch.device("cuda:0")
    amax = torch.full((4,), 7.0, device=dev)
    c = torch.full((64 * 32,), 5.0, device=dev)
    # K = 0: an empty sum, C = 0 and Amax = 0
    lib.mxgemm_amax(None, None, None, None, c, amax, 64, 32, 0, 1, 32, E4, E4)
    torch.cuda.synchronize()
    assert torch.all(c == 0).item() and amax[0].item() == 0.0
    # M = 0: nothing to compute, Amax = 0
    amax.fill_(7.0)
    lib.mxgemm_amax(None, None, None, None, None, amax, 0, 32, 64, 1, 32, E4, E4)
    torch.cuda.synchronize()
    assert amax[0].item() == 0.0


def test_host_pointer_rejected(lib):
    p = W.make_problem(128, 128, 128, 1, 32, E4, E4, seed=16)
    d = to_device(p)
    host_c = torch.empty(128 * 128, dtype=torch.float32, pin_memory=False)
    with pytest.raises(lib.MxgemmRuntimeError):
        lib.mxgemm_amax(d["A"], d["B"], d["SFA"], d["SFB"], host_c, d["Amax"], 128, 128, 128, 1, 32, E4, E4)


def test_high_level_wrapper_logical_sf(lib):
    M, N, K, L, sf = 256, 192, 256, 2, 32
    p = W.make_problem(M, N, K, L, sf, E4, E4, seed=17)
    dev = torch.device("cuda:0")
    a = torch.from_numpy(p["A"]).to(dev).view(torch.float8_e4m3fn).permute(1, 2, 0)   # (M, K, L) k-major
    b = torch.from_numpy(p["B"]).to(dev).view(torch.float8_e4m3fn).permute(1, 2, 0)
    mnb_a, mnb_b, kg = M // 128, -(-N // 128), K // (4 * sf)
    sfa = torch.from_numpy(p["SFA"]).to(dev).view(L, mnb_a, kg, 32, 4, 4).permute(3, 4, 1, 5, 2, 0)
    sfb = torch.from_numpy(p["SFB"]).to(dev).view(torch.float8_e8m0fnu).view(L, mnb_b, kg, 32, 4, 4)
    c, amax = lib.gemm_amax(a, b, sfa, sfb, sf_vec_size=sf)
    torch.cuda.synchronize()
    assert tuple(c.shape) == (M, N, L) and c.stride() == (N, 1, M * N)
    c_ref, s_ref, amax_ref = _oracle_full(p)
    check_c(c.permute(2, 0, 1).cpu().numpy(), c_ref, s_ref, "wrapper")
    check_amax(amax.item(), amax_ref)


@pytest.mark.parametrize("tile", ["t128", "t256"])
@pytest.mark.parametrize("sf", [32, 16])
def test_special_scale_bytes(lib, sf, tile):
    # E8M0 0xFF is NaN: every element of its block dequantises to NaN, so the
    # row's C is NaN and so is Amax.  E8M0 0x00 is 2^-127: its block's products
    # vanish below the absolute tolerance.  The bytes are set through the
    # oracle's logical view of the atoms.
    from oracle.sf_atom import sf_logical_view
    M, N, K, L = 300, 264, 384, 1
    p = W.make_problem(M, N, K, L, sf, E4, E4, seed=18)
    lva = sf_logical_view(p["SFA"], M, K, L, sf)
    nan_row, zero_row = 133, 7
    for m, kb, byte in ((nan_row, 5, 255), (zero_row, 2, 0), (zero_row, 3, 0)):
        lva[m % 32, (m // 32) % 4, m // 128, kb % 4, kb // 4, 0] = byte
    d = to_device(p)
    run(lib, p, d, flags=TILES[tile])
    c, amax = fetch(p, d)
    c_ref, s_ref, amax_ref = _oracle_full(p)
    assert np.isnan(c_ref[0, nan_row]).all() and np.isnan(amax_ref)
    nan_gpu = np.isnan(c)
    assert np.array_equal(nan_gpu, np.isnan(c_ref)), f"NaN rows differ: {np.argwhere(nan_gpu != np.isnan(c_ref))[:5]}"
    assert np.isnan(amax)
    keep = ~np.isnan(c_ref)
    check_c(c[keep], c_ref[keep], s_ref[keep], "special scale bytes")


@pytest.mark.parametrize("M,N,K,sf", [(2048, 2048, 2048, 32),    # 128x128 tiles, one workgroup per CU
                                      (256, 24576, 1536, 32),    # 128x128 tiles, two per CU
                                      (1000, 772, 1040, 16),     # a few 128x128 tiles
                                      (4000, 4100, 208, 16),     # 256x256 tiles, two K steps
                                      (4096, 4096, 4096, 32)])   # 256x256 tiles, several per workgroup
def test_back_to_back_calls_bitwise_equal(lib, M, N, K, sf):
    # Calls queued back to back on one stream, with a different problem in
    # between, must give bitwise the same C and Amax: a race inside a call
    # (LDS read before its DMA landed) or anything a call leaves in flight
    # shows up as a difference between repeats.
    print(f"back-to-back {M}x{N}x{K} sf={sf} config={lib.mxgemm_launch_config(M, N, K, 1, sf)}", flush=True)
    p = W.make_problem(M, N, K, 1, sf, E4, E4, seed=19)
    q = W.make_problem(384, 640, 512, 1, 32, E5, E4, seed=20)
    d, e = to_device(p), to_device(q)
    outs = []
    for _ in range(3):
        run(lib, p, d)
        run(lib, q, e)
        c, amax = fetch(p, d)
        outs.append((c.copy(), amax))
    for c, amax in outs[1:]:
        assert np.array_equal(c.view(np.uint32), outs[0][0].view(np.uint32))
        assert float_bits(amax) == float_bits(outs[0][1])
    rows = np.array([0, 1, M // 2, M - 1])
    c_ref, s_ref = oracle.gemm_rows(p["A"], p["B"], p["SFA"], p["SFB"], M, N, K, 1, sf, E4, E4, 0, rows)
    check_c(outs[0][0][0, rows], c_ref, s_ref, "back-to-back rows")


@pytest.mark.parametrize("M,N,K,L,sf,fa,fb", [
    (300, 520, 592, 2, 32, E4, E4),
    (1000, 772, 1040, 1, 16, E5, E4),
    # more 128x128 tiles (544) than workgroups: the operand stream runs on
    # across tiles, with one K step per tile and with a ragged eighth
    (2100, 4000, 112, 1, 32, E4, E4),
    (2100, 4000, 1008, 1, 16, E5, E4),
])
def test_tile_sizes_agree_bitwise(lib, M, N, K, L, sf, fa, fb):
    # Both tile sizes run the same per-output computation (the same K order
    # through the same MFMA slices), so their C and Amax agree bit for bit.
    p = W.make_problem(M, N, K, L, sf, fa, fb, seed=23)
    d = to_device(p)
    run(lib, p, d, flags=TILES["t128"])
    c128, a128 = fetch(p, d)
    c128 = c128.copy()
    run(lib, p, d, flags=TILES["t256"])
    c256, a256 = fetch(p, d)
    assert np.array_equal(c128.view(np.uint32), c256.view(np.uint32))
    assert float_bits(a128) == float_bits(a256)


@pytest.mark.parametrize("M,N,K,L", [
    (4000, 7168, 2048, 1),      # 448 tiles of 256x256: two rounds of 224
    (8192, 24576, 1536, 1),     # 3072 tiles: twelve whole rounds
    (2048, 2048, 2048, 1),      # 256 tiles of 128x128: one round
    (1024, 1024, 128, 1),       # 64 tiles: fewer than the CUs
    (2100, 4000, 112, 1),       # 544 tiles of 128x128: three rounds
    (4096, 4096, 4096, 8),      # batched: 8 x 256 tiles of 256x256
])
def test_persistent_grid_is_balanced(lib, M, N, K, L):
    # The persistent grid: the tile count when it fits the CUs; above that, the
    # same number of rounds as a full grid, with the workgroups of a round
    # rounded up to a multiple of 8 (so each XCD gets a contiguous run), so that
    # every workgroup runs the same number of tiles give or take one.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tm, tn, grid = lib.mxgemm_launch_config(M, N, K, L, 32)
    tiles = L * -(-M // tm) * -(-N // tn)
    if tiles <= cus:
        assert grid == tiles
    else:
        assert grid <= cus and grid % 8 == 0
        assert -(-tiles // grid) == -(-tiles // cus), "as many rounds as a full grid"
        per = [len(range(w, tiles, grid)) for w in range(grid)]
        assert max(per) - min(per) <= 1
