"""m-major C ("GEMM + Amax (SM100)", section "Parameters": C of shape (M, N, L)
with strides (1, M, M*N), the wrapper's c_major="m") on the GPU: against the
fp64 oracle within the stated tolerance, against the library's own n-major C
(the same sums, only the store layout and the MFMA operand order differ),
the guard band past C, K = 0, packed FP4 operands, the high-level wrapper, and
the projection workload sampled row by row."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import check_amax, check_c

pytestmark = pytest.mark.gpu

E4, E5, E2M1 = W.FMT_E4M3, W.FMT_E5M2, W.FMT_E2M1


@pytest.fixture(scope="module")
def lib():
    import block_scaled_precision_e4m3_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return lib


def run(lib, p, flags, guard=2048):
    """One call into a C buffer with a guard band; returns C as (L, M, N) float32 numpy and Amax."""
    M, N, K, L = p["M"], p["N"], p["K"], p["L"]
    dev = torch.device("cuda:0")
    A, B, SFA, SFB = (torch.from_numpy(np.ascontiguousarray(p[k])).to(dev) for k in ("A", "B", "SFA", "SFB"))
    buf = torch.full((L * M * N + guard,), -5.0, dtype=torch.float32, device=dev)
    am = torch.zeros(1, dtype=torch.float32, device=dev)
    lib.mxgemm_amax_ex(A, B, SFA, SFB, buf, am, M, N, K, L, p["sf"], p["a_fmt"], p["b_fmt"], flags)
    torch.cuda.synchronize()
    assert torch.all(buf[L * M * N:] == -5.0), "write past C"
    c = buf[:L * M * N].cpu().numpy()
    if flags & lib.MXG_FLAG_C_MMAJOR:
        c = c.reshape(L, N, M).transpose(0, 2, 1)
    else:
        c = c.reshape(L, M, N)
    return np.ascontiguousarray(c), float(am.item())


SHAPES = [
    (300, 520, 592, 2, 32, E4, E4),     # ragged M and N, K tail, two batches
    (256, 260, 336, 1, 16, E5, E4),     # sf=16, ragged N
    (1000, 772, 1040, 1, 16, E4, E5),
    (4000, 4100, 208, 1, 16, E5, E4),   # many tiles, ragged both ways
    (64, 36, 48, 3, 32, E4, E4),        # one partial tile per batch
]


@pytest.mark.parametrize("tile", [4, 8])       # 128x128, 256x256 tiles
@pytest.mark.parametrize("M,N,K,L,sf,fa,fb", SHAPES)
def test_mmajor_matches_oracle_and_nmajor(lib, M, N, K, L, sf, fa, fb, tile):
    print(f"m-major {M}x{N}x{K}x{L} sf={sf} tile flag {tile}", flush=True)
    p = W.make_problem(M, N, K, L, sf, fa, fb, seed=M + 3 * N + K)
    c_m, amax_m = run(lib, p, lib.MXG_FLAG_C_MMAJOR | tile)
    c_ref, s_ref, amax_ref = oracle.gemm_amax(p["A"], p["B"], p["SFA"], p["SFB"], M, N, K, L, sf, fa, fb)
    check_c(c_m, c_ref, s_ref, "m-major C")
    check_amax(amax_m, amax_ref)
    assert amax_m == float(np.max(np.abs(c_m)))
    # the n-major result of the same kernel holds the same sums
    c_n, amax_n = run(lib, p, tile)
    assert np.array_equal(c_m.view(np.uint32), c_n.view(np.uint32))
    assert amax_m == amax_n


def test_mmajor_k_zero(lib):
    p = W.make_problem(128, 96, 0, 2, 32, E4, E4, seed=3)
    c, amax = run(lib, p, lib.MXG_FLAG_C_MMAJOR)
    assert np.all(c == 0.0) and amax == 0.0


def test_mmajor_fp4_operands(lib):
    M, N, K, L = 300, 520, 544, 2
    p = W.make_problem(M, N, K, L, 32, E2M1, E2M1, seed=21)
    c_m, amax_m = run(lib, p, lib.MXG_FLAG_C_MMAJOR)
    c_ref, s_ref, amax_ref = oracle.gemm_amax(p["A"], p["B"], p["SFA"], p["SFB"], M, N, K, L, 32, E2M1, E2M1)
    check_c(c_m, c_ref, s_ref, "m-major C, FP4 operands")
    check_amax(amax_m, amax_ref)
    c_n, _ = run(lib, p, 0)
    assert np.array_equal(c_m.view(np.uint32), c_n.view(np.uint32))


def test_mmajor_wrapper_strides(lib):
    M, N, K, L, sf = 256, 192, 256, 2, 32
    p = W.make_problem(M, N, K, L, sf, E4, E4, seed=22)
    dev = torch.device("cuda:0")
    a = torch.from_numpy(p["A"]).to(dev).view(torch.float8_e4m3fn).permute(1, 2, 0)   # (M, K, L) k-major
    b = torch.from_numpy(p["B"]).to(dev).view(torch.float8_e4m3fn).permute(1, 2, 0)
    sfa, sfb = torch.from_numpy(p["SFA"]).to(dev), torch.from_numpy(p["SFB"]).to(dev)
    c, amax = lib.gemm_amax(a, b, sfa, sfb, sf_vec_size=sf, c_major="m")
    torch.cuda.synchronize()
    assert tuple(c.shape) == (M, N, L) and c.stride() == (1, M, M * N)
    c_ref, s_ref, amax_ref = oracle.gemm_amax(p["A"], p["B"], p["SFA"], p["SFB"], M, N, K, L, sf, E4, E4)
    check_c(c.permute(2, 0, 1).cpu().numpy(), c_ref, s_ref, "wrapper, m-major")
    check_amax(amax.item(), amax_ref)
    with pytest.raises(lib.MxgemmValueError):
        lib.gemm_amax(a, b, sfa, sfb, sf_vec_size=sf, c_major="m", c_dtype=torch.bfloat16)


def test_mmajor_projection_workload_rows(lib):
    # the projection workload at full size, m-major: sampled rows against the oracle
    p = W.make_workload(5)
    M, N, K, L, sf = p["M"], p["N"], p["K"], p["L"], p["sf"]
    c, amax = run(lib, p, lib.MXG_FLAG_C_MMAJOR, guard=0)
    rows = np.array([0, 1, 255, 256, 4097, M - 1])
    c_ref, s_ref = oracle.gemm_rows(p["A"], p["B"], p["SFA"], p["SFB"], M, N, K, L, sf, p["a_fmt"], p["b_fmt"], 0,
                                    rows)
    check_c(c[0, rows], c_ref, s_ref, "projection, m-major rows")
    assert amax == float(np.max(np.abs(c)))


# --- m-major A / n-major B: codes rewritten k-major by mxgemm_codes_to_kmajor --------

@pytest.mark.parametrize("MN,K,L", [(64, 64, 1), (80, 48, 3), (4096, 1536, 1), (1040, 208, 2), (16, 16, 1)])
def test_codes_to_kmajor_bit_exact(lib, MN, K, L):
    print(f"codes_to_kmajor {MN}x{K}x{L}", flush=True)
    rng = np.random.default_rng(MN + K + L)
    src = rng.integers(0, 256, size=(L, K, MN), dtype=np.uint8)
    dev = torch.device("cuda:0")
    s = torch.from_numpy(src).to(dev)
    guard = 4096
    d = torch.full((L * MN * K + guard,), 0xA5, dtype=torch.uint8, device=dev)
    lib.codes_to_kmajor(s, d, MN, K, L)
    torch.cuda.synchronize()
    out = d.cpu().numpy()
    assert np.all(out[L * MN * K:] == 0xA5), "write past the destination"
    assert np.array_equal(out[:L * MN * K].reshape(L, MN, K), src.transpose(0, 2, 1))


@pytest.mark.parametrize("a_major,b_major", [("m", "k"), ("k", "n"), ("m", "n")])
def test_mmajor_operands_through_wrapper(lib, a_major, b_major):
    M, N, K, L, sf = 320, 272, 384, 2, 32
    p = W.make_problem(M, N, K, L, sf, E4, E5, seed=23)
    dev = torch.device("cuda:0")

    def view(codes, dtype, major):
        # codes (L, rows, K) -> the pages' (rows, K, L) view: k-major as stored, or m/n-major
        t = torch.from_numpy(np.ascontiguousarray(codes)).to(dev).view(dtype)
        if major == "k":
            return t.permute(1, 2, 0)
        mm = t.permute(0, 2, 1).contiguous()           # (L, K, rows), rows contiguous
        return mm.permute(2, 1, 0)                     # (rows, K, L) with strides (1, rows, rows*K)

    a = view(p["A"], torch.float8_e4m3fn, a_major)
    b = view(p["B"], torch.float8_e5m2, b_major)
    if a_major == "m":
        assert a.stride() == (1, M, M * K)
    sfa, sfb = torch.from_numpy(p["SFA"]).to(dev), torch.from_numpy(p["SFB"]).to(dev)
    c, amax = lib.gemm_amax(a, b, sfa, sfb, sf_vec_size=sf)
    ck, amaxk = lib.gemm_amax(view(p["A"], torch.float8_e4m3fn, "k"), view(p["B"], torch.float8_e5m2, "k"),
                              sfa, sfb, sf_vec_size=sf)
    torch.cuda.synchronize()
    assert torch.equal(c, ck) and torch.equal(amax, amaxk)
    c_ref, s_ref, amax_ref = oracle.gemm_amax(p["A"], p["B"], p["SFA"], p["SFB"], M, N, K, L, sf, E4, E5)
    check_c(c.permute(2, 0, 1).cpu().numpy(), c_ref, s_ref, f"A {a_major}-major, B {b_major}-major")
    check_amax(amax.item(), amax_ref)
