"""A seeded sweep over the GEMM's option space, every output against the fp64 oracle.

Ninety problems drawn from one seeded generator: ragged M and N (N a
multiple of 4), K a multiple of 16 with and without a tail past the last
128-element step, one to three batches, sf 16 or 32, every 8-bit format
pair, the automatic tile choice or either tile forced, and one of: plain
n-major C, m-major C, m-major A, n-major B, both, Amax accumulated into a
preset value above or below the result, or a bfloat16 / float16 C ("GEMM +
Amax (SM100)", sections "Equations" and "Parameters").  Each case checks
every C element and Amax against the oracle at the stated tolerance (a
16-bit C: bit for bit the round-to-nearest-even of the library's float32 C,
which meets the tolerance), and that nothing past C was written.  Thirty
more draw packed FP4 (E2M1) operands, with the modes FP4 takes (K a multiple
of 32; no 256x256 tiles at sf = 16; k-major operands).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import AMAX_REL, TOL_ABS, TOL_REL

pytestmark = pytest.mark.gpu
E4, E5 = W.FMT_E4M3, W.FMT_E5M2
MODES = ["plain", "c_mmajor", "a_mmajor", "b_nmajor", "ab_major", "accumulate_up", "accumulate_down", "c_bf16",
         "c_f16"]


def _cases(n=90, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        mode = MODES[i % len(MODES)]
        M = int(rng.integers(1, 521))
        N = 4 * int(rng.integers(1, 131))
        K = 16 * int(rng.integers(1, 51))
        L = int(rng.choice([1, 1, 2, 3]))
        if mode == "c_mmajor":
            M = 4 * max(1, M // 4)
        if mode in ("a_mmajor", "ab_major"):
            M = 16 * max(1, M // 16)
        if mode in ("b_nmajor", "ab_major"):
            N = 16 * max(1, N // 16)
        sf = int(rng.choice([16, 32]))
        fa, fb = int(rng.choice([E4, E5])), int(rng.choice([E4, E5]))
        tile = int(rng.choice([0, 4, 8]))
        out.append((i, mode, M, N, K, L, sf, fa, fb, tile))
    return out


CASES = _cases()
FP4_MODES = ["plain", "c_mmajor", "accumulate_down", "c_bf16", "accumulate_up"]


def _fp4_cases(n=30, seed=4048):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        mode = FP4_MODES[i % len(FP4_MODES)]
        M = int(rng.integers(1, 521))
        if mode == "c_mmajor":
            M = 4 * max(1, M // 4)
        N = 4 * int(rng.integers(1, 131))
        K = 32 * int(rng.integers(1, 40))
        L = int(rng.choice([1, 1, 2]))
        sf = int(rng.choice([16, 32]))
        tile = int(rng.choice([0, 4] if sf == 16 else [0, 4, 8]))
        out.append((100 + i, mode, M, N, K, L, sf, W.FMT_E2M1, W.FMT_E2M1, tile))
    return out


FP4_CASES = _fp4_cases()


@pytest.fixture(scope="module")
def lib():
    import block_scaled_precision_e4m3_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return lib


@pytest.mark.parametrize("i,mode,M,N,K,L,sf,fa,fb,tile", CASES + FP4_CASES)
def test_sweep_against_oracle(lib, i, mode, M, N, K, L, sf, fa, fb, tile):
    print(f"sweep case {i}: {mode} {M}x{N}x{K}x{L} sf={sf} fmts {fa},{fb} tile flag {tile}", flush=True)
    p = W.make_problem(M, N, K, L, sf, fa, fb, seed=1000 + i, dist="student_t3" if i % 2 else "normal")
    c_ref, s_ref, a_ref = oracle.gemm_amax(p["A"], p["B"], p["SFA"], p["SFB"], M, N, K, L, sf, fa, fb)
    dev = torch.device("cuda:0")
    a_mm = mode in ("a_mmajor", "ab_major")
    b_mm = mode in ("b_nmajor", "ab_major")
    A = torch.from_numpy(np.ascontiguousarray(p["A"].transpose(0, 2, 1) if a_mm else p["A"])).to(dev)
    B = torch.from_numpy(np.ascontiguousarray(p["B"].transpose(0, 2, 1) if b_mm else p["B"])).to(dev)
    SFA, SFB = torch.from_numpy(p["SFA"]).to(dev), torch.from_numpy(p["SFB"]).to(dev)
    guard = 4096
    buf = torch.full((L * M * N + guard,), -7.0, dtype=torch.float32, device=dev)
    preset = {"accumulate_up": 2.0 * a_ref, "accumulate_down": 0.5 * a_ref}.get(mode, -1.0)
    am = torch.full((4,), preset, dtype=torch.float32, device=dev)
    flags = tile
    flags |= lib.MXG_FLAG_C_MMAJOR if mode == "c_mmajor" else 0
    flags |= lib.MXG_FLAG_A_MMAJOR if a_mm else 0
    flags |= lib.MXG_FLAG_B_NMAJOR if b_mm else 0
    flags |= lib.MXG_FLAG_AMAX_ACCUMULATE if mode.startswith("accumulate") else 0
    lib.mxgemm_amax_ex(A, B, SFA, SFB, buf, am, M, N, K, L, sf, fa, fb, flags)
    torch.cuda.synchronize()
    assert torch.all(buf[L * M * N:] == -7.0), "write past C"
    if mode in ("c_bf16", "c_f16"):
        dt = torch.bfloat16 if mode == "c_bf16" else torch.float16
        buf16 = torch.full((L * M * N + guard,), -7.0, dtype=dt, device=dev)
        am16 = torch.full((4,), -1.0, dtype=torch.float32, device=dev)
        f16 = lib.MXG_FLAG_C_BF16 if mode == "c_bf16" else lib.MXG_FLAG_C_F16
        lib.mxgemm_amax_ex(A, B, SFA, SFB, buf16, am16, M, N, K, L, sf, fa, fb, flags | f16)
        torch.cuda.synchronize()
        assert torch.all(buf16[L * M * N:] == -7.0), "write past the 16-bit C"
        assert torch.equal(buf16[:L * M * N].view(torch.int16), buf[:L * M * N].to(dt).view(torch.int16))
        assert torch.equal(am16, am)
    c = buf[:L * M * N].double().cpu().numpy()
    c = c.reshape(L, N, M).transpose(0, 2, 1) if mode == "c_mmajor" else c.reshape(L, M, N)
    bad = ~(np.abs(c - c_ref) <= TOL_REL * s_ref + TOL_ABS)
    assert not bad.any(), f"{int(bad.sum())} outputs outside tolerance, first at {np.argwhere(bad)[0].tolist()}"
    got = float(am[0])
    if mode == "accumulate_up":
        assert got == np.float32(preset), "accumulate: a larger preset Amax must stay"
    else:
        assert abs(got - a_ref) <= AMAX_REL * a_ref, f"amax {got} against {a_ref}"
