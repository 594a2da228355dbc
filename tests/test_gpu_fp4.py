"""Packed FP4 (E2M1) operands on the GPU against the oracle: ragged shapes,
batches, 16-bit C, the guard band past C, the error rules, and a large shape
sampled row by row."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

E2M1 = W.FMT_E2M1


@pytest.fixture(scope="module")
def lib():
    import block_scaled_precision_e4m3_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return lib


def run(lib, p, flags=0, c_dtype=torch.float32, guard=2048):
    M, N, K, L, sf = p["M"], p["N"], p["K"], p["L"], p["sf"]
    dev = torch.device("cuda:0")
    A, B, SFA, SFB = (torch.from_numpy(np.ascontiguousarray(p[k])).to(dev) for k in ("A", "B", "SFA", "SFB"))
    buf = torch.full((L * M * N + guard,), -5.0, dtype=c_dtype, device=dev)
    am = torch.zeros(1, dtype=torch.float32, device=dev)
    lib.mxgemm_amax_ex(A, B, SFA, SFB, buf, am, M, N, K, L, sf, E2M1, E2M1, flags)
    torch.cuda.synchronize()
    assert torch.all(buf[L * M * N:] == -5.0), "write past C"
    return buf[:L * M * N], am


@pytest.mark.parametrize("sf,tile", [(32, 0), (32, 4), (32, 8), (16, 0), (16, 4)])  # tile flag: auto, 128, 256
@pytest.mark.parametrize("shape", [(256, 256, 256, 1), (300, 520, 544, 2), (64, 100, 32, 1), (520, 260, 1536, 1),
                                   (256, 256, 0, 1)])
def test_fp4_matches_oracle(lib, shape, sf, tile):
    M, N, K, L = shape
    print(f"fp4 {shape} sf {sf} tile flag {tile}", flush=True)
    p = W.make_problem(M, N, K, L, sf, E2M1, E2M1, seed=M + N + K + sf + 1)
    c, am = run(lib, p, tile)
    cref, sref, aref = oracle.gemm_amax(p["A"], p["B"], p["SFA"], p["SFB"], M, N, K, L, sf, E2M1, E2M1)
    got = c.view(L, M, N).double().cpu().numpy()
    assert np.all(np.abs(got - cref) <= 1e-5 * sref + 1e-30)
    assert abs(float(am) - aref) <= 1e-5 * aref


@pytest.mark.parametrize("sf", [32, 16])
def test_fp4_16bit_c_is_rne_of_f32(lib, sf):
    p = W.make_problem(300, 260, 512, 1, sf, E2M1, E2M1, seed=5)
    c32, a32 = run(lib, p)
    c16, a16 = run(lib, p, lib.MXG_FLAG_C_BF16, torch.bfloat16)
    assert torch.equal(c16.view(torch.int16), c32.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(a16, a32)


def test_fp4_sf16_m_major_c_is_the_transpose(lib):
    # the m-major C of the 128x128 kernel at sf = 16 holds exactly the n-major C transposed
    M, N, K = 260, 384, 640
    p = W.make_problem(M, N, K, 1, 16, E2M1, E2M1, seed=21)
    cn, an = run(lib, p)
    cm, am = run(lib, p, lib.MXG_FLAG_C_MMAJOR)
    assert torch.equal(cm.view(N, M).t(), cn.view(M, N))
    assert torch.equal(am, an)


def test_fp4_sf16_ragged_k_and_scale_tail(lib):
    # K = 32 and 96: the last step holds one or three 16-element blocks of the four an atom covers;
    # the oracle expands the atoms on its own
    for M, N, K in ((130, 260, 32), (257, 131 * 4, 96)):
        p = W.make_problem(M, N, K, 1, 16, E2M1, E2M1, seed=K + 3)
        c, am = run(lib, p)
        cref, sref, aref = oracle.gemm_amax(p["A"], p["B"], p["SFA"], p["SFB"], M, N, K, 1, 16, E2M1, E2M1)
        got = c.view(1, M, N).double().cpu().numpy()
        assert np.all(np.abs(got - cref) <= 1e-5 * sref + 1e-30), (M, N, K)
        assert abs(float(am) - aref) <= 1e-5 * aref


def test_fp4_large_sampled(lib):
    # the projection workload's shape with FP4 operands; rows sampled against the oracle
    M, N, K = 8192, 24576, 1536
    print("fp4 projection shape", flush=True)
    p = W.make_problem(M, N, K, 1, 32, E2M1, E2M1, seed=9, b_scale=float(1.0 / np.sqrt(K)))
    c, am = run(lib, p, guard=1 << 16)
    rows = np.array([0, 1, 255, 256, 4097, M - 1])
    cref, sref = oracle.gemm_rows(p["A"], p["B"], p["SFA"], p["SFB"], M, N, K, 1, 32, E2M1, E2M1, 0, rows)
    got = c.view(M, N)[rows].double().cpu().numpy()
    assert np.all(np.abs(got - cref) <= 1e-5 * sref + 1e-30)
    assert float(am) == float(torch.max(torch.abs(c)))


def test_fp4_rules(lib):
    ok = lib.mxgemm_check_support
    assert ok(256, 256, 256, 1, 32, E2M1, E2M1) == lib.MXG_OK
    assert ok(256, 256, 256, 1, 16, E2M1, E2M1) == lib.MXG_OK
    assert ok(256, 256, 256, 1, 8, E2M1, E2M1) == lib.MXG_ERR_SFVEC
    assert ok(256, 256, 256, 1, 32, E2M1, 0) == lib.MXG_ERR_FMT
    assert ok(256, 256, 240, 1, 32, E2M1, E2M1) == lib.MXG_ERR_ALIGN
    p = W.make_problem(128, 128, 128, 1, 32, E2M1, E2M1, seed=1)
    with pytest.raises(ValueError):
        run(lib, p, lib.MXG_FLAG_FP8_MFMA)
    p16 = W.make_problem(128, 128, 128, 1, 16, E2M1, E2M1, seed=1)
    with pytest.raises(ValueError):
        run(lib, p16, lib.MXG_FLAG_TILE_256)   # sf = 16 runs 128x128 tiles only
