"""Plans (mxgemm_plan_init / mxgemm_plan_execute) give bitwise the results of
mxgemm_amax_ex with the same sizes and flags, across tile kernels, C types,
Amax accumulation and repeated use."""

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

E4, E5 = W.FMT_E4M3, W.FMT_E5M2


@pytest.fixture(scope="module")
def lib():
    import block_scaled_precision_e4m3_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return lib


@pytest.mark.parametrize("flags", [0, 4, 8, 32, 64, 2, 1, 128, 128 | 1])
def test_plan_matches_direct_call(lib, flags):
    M, N, K, L, sf = 300, 520, 256, 2, 16
    p = W.make_problem(M, N, K, L, sf, E5, E4, seed=21)
    print(f"plan flags={flags}", flush=True)
    dev = torch.device("cuda:0")
    A, B, SFA, SFB = (torch.from_numpy(p[k]).to(dev) for k in ("A", "B", "SFA", "SFB"))
    dt = torch.bfloat16 if flags & 32 else torch.float16 if flags & 64 else torch.float32
    outs = []
    for use_plan in (False, True):
        C = torch.full((L * M * N,), -3.0, dtype=dt, device=dev)
        am = torch.full((1,), 0.5, dtype=torch.float32, device=dev)   # accumulate starts from 0.5
        if use_plan:
            plan = lib.Plan(M, N, K, L, sf, E5, E4, flags)
            plan(A, B, SFA, SFB, C, am)
            plan(A, B, SFA, SFB, C, am)   # a plan is reusable
        else:
            lib.mxgemm_amax_ex(A, B, SFA, SFB, C, am, M, N, K, L, sf, E5, E4, flags)
            lib.mxgemm_amax_ex(A, B, SFA, SFB, C, am, M, N, K, L, sf, E5, E4, flags)
        torch.cuda.synchronize()
        outs.append((C, am))
    assert torch.equal(outs[0][0].view(torch.uint8), outs[1][0].view(torch.uint8))
    assert torch.equal(outs[0][1], outs[1][1])


def test_plan_pointer_checks(lib):
    p = W.make_problem(128, 128, 128, 1, 32, E4, E4, seed=2)
    dev = torch.device("cuda:0")
    A, B, SFA, SFB = (torch.from_numpy(p[k]).to(dev) for k in ("A", "B", "SFA", "SFB"))
    C = torch.empty(128 * 128 + 8, dtype=torch.float32, device=dev)
    am = torch.zeros(4, dtype=torch.float32, device=dev)
    plan = lib.Plan(128, 128, 128, 1, 32, E4, E4)
    with pytest.raises(ValueError):
        plan(A, B, SFA, SFB, C.data_ptr() + 4, am)     # C not 16-byte aligned
    with pytest.raises(ValueError):
        plan(A, None, SFA, SFB, C, am)
