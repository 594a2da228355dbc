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


@pytest.mark.parametrize("M,N,K,sf,fa,fb", [(1000, 772, 512, 16, E5, E4),     # 128x128 kernel
                                            (4096, 4100, 384, 32, E4, E4)])   # 256x256 kernel
def test_plan_captured_in_a_graph(lib, M, N, K, sf, fa, fb):
    # A plan call (the Amax clearing kernel, then the GEMM; no memset node) is
    # captured into a graph on a side stream and replayed several times, with
    # eager work and synchronisation between replays; every replay must give
    # bitwise the result of a direct call.
    print(f"graph capture {M}x{N}x{K} sf={sf}", flush=True)
    L = 1
    p = W.make_problem(M, N, K, L, sf, fa, fb, seed=22)
    dev = torch.device("cuda:0")
    A, B, SFA, SFB = (torch.from_numpy(p[k]).to(dev) for k in ("A", "B", "SFA", "SFB"))
    plan = lib.Plan(M, N, K, L, sf, fa, fb)
    C_ref = torch.empty(L * M * N, dtype=torch.float32, device=dev)
    am_ref = torch.full((4,), -1.0, dtype=torch.float32, device=dev)
    plan(A, B, SFA, SFB, C_ref, am_ref)
    torch.cuda.synchronize()

    C = torch.full((L * M * N,), float("nan"), dtype=torch.float32, device=dev)
    am = torch.full((4,), -1.0, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        plan(A, B, SFA, SFB, C, am, stream=side)
    torch.cuda.synchronize()
    for rep in range(4):
        C.fill_(float("nan"))
        am.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int32), C_ref.view(torch.int32)), f"replay {rep}: C differs"
        assert torch.equal(am[:1], am_ref[:1]), f"replay {rep}: Amax differs"
    # the graph's inputs are read at replay time: new A gives the new result
    A2 = A ^ 0x80                       # every A sign flipped
    A.copy_(A2)
    plan(A, B, SFA, SFB, C_ref, am_ref)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int32), C_ref.view(torch.int32))
