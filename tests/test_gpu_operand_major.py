"""m-major A and n-major B read by the GEMM itself ("GEMM + Amax (SM100)",
section "Parameters": A strides (1, M, M*K), B strides (1, N, N*K)).

The kernel stages such a tile as K rows in LDS and reads it with the
transposing LDS load into the same registers the k-major path fills, so C and
Amax must equal bit for bit those of the same codes stored k-major; both are
also checked against the oracle.  Ragged M and N (multiples of 16, not of
the tile), K tails, batches, both tile sizes, both block sizes and all format
pairs; the projection workload at full size; a guard band past C; the rules.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
E4, E5 = W.FMT_E4M3, W.FMT_E5M2


@pytest.fixture(scope="module")
def lib():
    import block_scaled_precision_e4m3_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return lib


def run(lib, p, mj, tile, guard=4096):
    """C and Amax of the problem with A m-major (mj bit 0) and/or B n-major (bit 1), through the C ABI."""
    M, N, K, L, sf = p["M"], p["N"], p["K"], p["L"], p["sf"]
    dev = torch.device("cuda:0")

    def operand(codes, mmajor):
        c = np.ascontiguousarray(codes.transpose(0, 2, 1) if mmajor else codes)
        return torch.from_numpy(c).to(dev)
    A = operand(p["A"], mj & 1)
    B = operand(p["B"], mj & 2)
    SFA, SFB = torch.from_numpy(p["SFA"]).to(dev), torch.from_numpy(p["SFB"]).to(dev)
    buf = torch.full((L * M * N + guard,), -7.0, dtype=torch.float32, device=dev)
    am = torch.zeros(1, dtype=torch.float32, device=dev)
    flags = tile | (lib.MXG_FLAG_A_MMAJOR if mj & 1 else 0) | (lib.MXG_FLAG_B_NMAJOR if mj & 2 else 0)
    lib.mxgemm_amax_ex(A, B, SFA, SFB, buf, am, M, N, K, L, sf, p["a_fmt"], p["b_fmt"], flags)
    torch.cuda.synchronize()
    assert torch.all(buf[L * M * N:] == -7.0), "write past C"
    return buf[:L * M * N], am


CASES = [
    # M, N, K, L, sf, a_fmt, b_fmt
    (256, 256, 256, 1, 32, E4, E4),
    (272, 400, 208, 2, 32, E4, E5),    # ragged M and N, K tail of 80, two batches
    (160, 96, 48, 1, 16, E5, E4),      # one short K step, sf = 16
    (528, 304, 1040, 1, 16, E5, E5),   # several K steps and a tail
    (16, 32, 16, 3, 32, E4, E4),       # tiny: one chunk of columns
]


@pytest.mark.parametrize("tile", [4, 8])        # 128x128 and 256x256 tiles
@pytest.mark.parametrize("mj", [1, 2, 3])       # A m-major, B n-major, both
@pytest.mark.parametrize("M,N,K,L,sf,fa,fb", CASES)
def test_operand_major_equals_k_major_and_oracle(lib, M, N, K, L, sf, fa, fb, mj, tile):
    print(f"operand majors {mj} {M}x{N}x{K}x{L} sf={sf} tile flag {tile}", flush=True)
    p = W.make_problem(M, N, K, L, sf, fa, fb, seed=M + 3 * N + 7 * K + L)
    c, am = run(lib, p, mj, tile)
    ck, amk = run(lib, p, 0, tile)
    assert torch.equal(c, ck), "m-major operands differ from the k-major result"
    assert torch.equal(am, amk)
    c_ref, s_ref, a_ref = oracle.gemm_amax(p["A"], p["B"], p["SFA"], p["SFB"], M, N, K, L, sf, fa, fb)
    got = c.view(L, M, N).double().cpu().numpy()
    assert np.all(np.abs(got - c_ref) <= 1e-5 * s_ref + 1e-30)
    assert abs(float(am) - a_ref) <= 1e-5 * a_ref


def test_operand_major_projection_workload(lib):
    # the projection workload at full size with both operands m/n-major: bitwise the k-major C
    print("operand majors: projection workload", flush=True)
    p = W.make_workload(5)
    c, am = run(lib, p, 3, 0, guard=1 << 16)
    ck, amk = run(lib, p, 0, 0, guard=1 << 16)
    assert torch.equal(c, ck) and torch.equal(am, amk)
    rows = np.array([0, 255, 4096, p["M"] - 1])
    c_ref, s_ref = oracle.gemm_rows(p["A"], p["B"], p["SFA"], p["SFB"], p["M"], p["N"], p["K"], 1, p["sf"],
                                    p["a_fmt"], p["b_fmt"], 0, rows)
    got = c.view(p["M"], p["N"])[rows].double().cpu().numpy()
    assert np.all(np.abs(got - c_ref) <= 1e-5 * s_ref + 1e-30)


def test_operand_major_plan(lib):
    # a plan carries the flags; two executions in a row give the direct call's result
    p = W.make_problem(272, 400, 208, 1, 32, E4, E5, seed=3)
    c, am = run(lib, p, 3, 0)
    dev = torch.device("cuda:0")
    A = torch.from_numpy(np.ascontiguousarray(p["A"].transpose(0, 2, 1))).to(dev)
    B = torch.from_numpy(np.ascontiguousarray(p["B"].transpose(0, 2, 1))).to(dev)
    SFA, SFB = torch.from_numpy(p["SFA"]).to(dev), torch.from_numpy(p["SFB"]).to(dev)
    plan = lib.Plan(272, 400, 208, 1, 32, E4, E5, lib.MXG_FLAG_A_MMAJOR | lib.MXG_FLAG_B_NMAJOR)
    for _ in range(2):
        C = torch.empty(272 * 400, dtype=torch.float32, device=dev)
        Am = torch.zeros(1, dtype=torch.float32, device=dev)
        plan(A, B, SFA, SFB, C, Am)
        torch.cuda.synchronize()
        assert torch.equal(C, c) and torch.equal(Am, am)


def test_operand_major_rules(lib):
    p = W.make_problem(264, 256, 128, 1, 32, E4, E4, seed=1)
    with pytest.raises(ValueError):
        run(lib, p, 1, 0)                        # M % 16 != 0 with A m-major
    q = W.make_problem(256, 256, 128, 1, 32, E4, E4, seed=1)
    dev = torch.device("cuda:0")
    A, B = torch.from_numpy(q["A"]).to(dev), torch.from_numpy(q["B"]).to(dev)
    SFA, SFB = torch.from_numpy(q["SFA"]).to(dev), torch.from_numpy(q["SFB"]).to(dev)
    C = torch.empty(256 * 256, dtype=torch.float32, device=dev)
    am = torch.zeros(1, dtype=torch.float32, device=dev)
    for bad in (lib.MXG_FLAG_FP8_MFMA, lib.MXG_FLAG_C_MMAJOR):
        with pytest.raises(ValueError):
            lib.mxgemm_amax_ex(A, B, SFA, SFB, C, am, 256, 256, 128, 1, 32, E4, E4, lib.MXG_FLAG_A_MMAJOR | bad)
