"""16-bit C (MXG_FLAG_C_BF16 / MXG_FLAG_C_F16): the 16-bit output equals, bit
for bit, torch's round-to-nearest-even conversion of the library's own float32
C for the same inputs (the accumulation is the same, only the epilogue's
rounding differs), the amax is the float32 one, nothing is written past C,
and the float32 C itself matches the oracle within the GEMM tolerance."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

E4, E5 = W.FMT_E4M3, W.FMT_E5M2
TILES = {"t128": 4, "t256": 8}


@pytest.fixture(scope="module")
def lib():
    import block_scaled_precision_e4m3_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return lib


def run(lib, p, flags, c_dtype, guard=4096):
    M, N, K, L = p["M"], p["N"], p["K"], p["L"]
    dev = torch.device("cuda:0")
    A, B, SFA, SFB = (torch.from_numpy(p[k]).to(dev) for k in ("A", "B", "SFA", "SFB"))
    buf = torch.full((L * M * N + guard,), -7.0, dtype=c_dtype, device=dev)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    lib.mxgemm_amax_ex(A, B, SFA, SFB, buf, amax, M, N, K, L, p["sf"], p["a_fmt"], p["b_fmt"], flags)
    torch.cuda.synchronize()
    assert torch.all(buf[L * M * N:] == -7.0), "write past C"
    return buf[:L * M * N], amax


@pytest.mark.parametrize("tile", list(TILES))
@pytest.mark.parametrize("cdt", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(256, 256, 256, 1, 32, E4, E4), (300, 260, 176, 2, 16, E5, E4),
                                   (520, 1028, 512, 1, 32, E4, E5)])
def test_c16_is_rne_of_c32(lib, shape, cdt, tile):
    M, N, K, L, sf, fa, fb = shape
    print(f"c16 {cdt} {tile} {shape}", flush=True)
    p = W.make_problem(M, N, K, L, sf, fa, fb, seed=M + N + K)
    flag = lib.MXG_FLAG_C_BF16 if cdt == "bf16" else lib.MXG_FLAG_C_F16
    dt = torch.bfloat16 if cdt == "bf16" else torch.float16
    c32, a32 = run(lib, p, TILES[tile], torch.float32)
    c16, a16 = run(lib, p, TILES[tile] | flag, dt)
    assert torch.equal(c16.view(torch.int16), c32.to(dt).view(torch.int16))
    assert torch.equal(a16, a32)
    # the float32 C against the oracle
    cref, sref, aref = oracle.gemm_amax(p["A"], p["B"], p["SFA"], p["SFB"], M, N, K, L, sf, fa, fb)
    got = c32.view(L, M, N).double().cpu().numpy()
    assert np.all(np.abs(got - cref) <= 1e-5 * sref + 1e-30)
    assert abs(float(a32) - aref) <= 1e-5 * aref


def test_f16_overflow_is_inf(lib):
    # scales push |C| past 65504: float16 C holds +-inf where torch's conversion does
    p = W.make_problem(256, 256, 256, 1, 32, E4, E4, seed=3)
    p["SFA"] = np.where(p["SFA"] == 127, 127, np.minimum(p["SFA"].astype(np.int32) + 14, 254)).astype(np.uint8)
    c32, a32 = run(lib, p, 0, torch.float32)
    c16, a16 = run(lib, p, lib.MXG_FLAG_C_F16, torch.float16)
    assert bool(torch.isinf(c16).any()), "test data should overflow float16"
    assert torch.equal(c16.view(torch.int16), c32.to(torch.float16).view(torch.int16))
    assert torch.equal(a16, a32) and bool(torch.isfinite(a32).all())


@pytest.mark.parametrize("cdt", ["bf16", "f16"])
def test_c16_projection_workload(lib, cdt):
    # the full projection shape on the 256x256 kernel, compared on the GPU
    p = W.make_workload(5)
    print(f"c16 {cdt} projection workload", flush=True)
    flag = lib.MXG_FLAG_C_BF16 if cdt == "bf16" else lib.MXG_FLAG_C_F16
    dt = torch.bfloat16 if cdt == "bf16" else torch.float16
    c32, a32 = run(lib, p, 0, torch.float32, guard=1 << 16)
    c16, a16 = run(lib, p, flag, dt, guard=1 << 16)
    assert torch.equal(c16.view(torch.int16), c32.to(dt).view(torch.int16))
    assert torch.equal(a16, a32)


def test_c16_flag_errors(lib):
    p = W.make_problem(128, 128, 128, 1, 32, E4, E4, seed=1)
    with pytest.raises(ValueError):
        run(lib, p, lib.MXG_FLAG_C_BF16 | lib.MXG_FLAG_C_F16, torch.bfloat16)
    with pytest.raises(ValueError):
        run(lib, p, lib.MXG_FLAG_C_BF16 | lib.MXG_FLAG_FP8_MFMA, torch.bfloat16)
