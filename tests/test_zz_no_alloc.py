"""The allocation-free projection entry (mxgemm_projection_mxfp8_noalloc).

It takes its workspace from the library's fixed per-device scratch array
instead of a caller buffer; everything else is the workspace entry
(mxgemm_projection_mxfp8), whose outputs are checked against the oracle in
test_gpu_proj_fused.py.  Two calls in a row, the second smaller, each must
equal the workspace entry's outputs bit for bit (the scratch still holds the
first call's atoms when the second runs), with guard bands past every output.
A problem whose workspace exceeds the scratch is refused before any work.
"""

import ctypes

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
E4 = W.FMT_E4M3
GUARD = 4096


@pytest.fixture(scope="module")
def lib():
    import block_scaled_precision_e4m3_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return lib


def problem(tokens, heads, d, qr, K, seed):
    rng = np.random.default_rng(seed)
    n = heads * d
    x = rng.standard_normal((1, tokens, K)).astype(np.float32)
    w = (rng.standard_normal((1, n, K)) / np.sqrt(K)).astype(np.float32)
    xq, xs = W.mx_quantize(x, 32, E4)
    wq, ws = W.mx_quantize(w, 32, E4)
    theta = rng.uniform(0, 2 * np.pi, size=(tokens, max(qr // 2, 1)))
    cs = np.concatenate([np.cos(theta), 0.75 * np.cos(theta)], axis=1)[:, :qr]
    sn = np.concatenate([np.sin(theta), -1.25 * np.sin(theta)], axis=1)[:, :qr]
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return (t(xq[0]), t(wq[0]), t(xs[0]), t(ws[0]),
            torch.from_numpy(cs.astype(np.float32)).to(torch.bfloat16).to(dev),
            torch.from_numpy(sn.astype(np.float32)).to(torch.bfloat16).to(dev))


def guarded_outputs(tokens, heads, d, fill):
    dev = torch.device("cuda:0")
    n = tokens * heads * d
    sizes = (n, n // 32, n, n // 32)
    bufs = [torch.full((s + GUARD,), fill, dtype=torch.uint8, device=dev) for s in sizes]
    return bufs, sizes


def c_abi_noalloc(lib, args, bufs, tokens, heads, d, qr, K):
    f = ctypes.CDLL(lib.LIB_PATH).mxgemm_projection_mxfp8_noalloc
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    f.argtypes = [vp] * 10 + [i64] * 5 + [vp]
    f.restype = ctypes.c_int
    ptrs = [a.data_ptr() for a in args] + [b.data_ptr() for b in bufs]
    return f(*ptrs, tokens, heads, d, qr, K, None)


@pytest.mark.parametrize("calls", [[(256, 128, 192, 64, 1536), (96, 4, 192, 64, 160)]])
def test_noalloc_equals_workspace_entry_on_two_calls(lib, calls):
    dev = torch.device("cuda:0")
    for i, (tokens, heads, d, qr, K) in enumerate(calls):
        print(f"no-alloc projection call {i}: {tokens} tokens, {heads}x{d}, qr={qr}, K={K}", flush=True)
        args = problem(tokens, heads, d, qr, K, seed=11 + i)
        bufs, sizes = guarded_outputs(tokens, heads, d, 0xA5)
        assert c_abi_noalloc(lib, args, bufs, tokens, heads, d, qr, K) == lib.MXG_OK
        torch.cuda.synchronize()
        for b, s in zip(bufs, sizes):
            assert torch.all(b[s:] == 0xA5).item(), "write past an output"
        need = lib._lib.mxgemm_projection_workspace_bytes(tokens, heads, d, K)
        assert need <= lib.MXGEMM_NOALLOC_SCRATCH_BYTES
        wsp = torch.full((need,), 0x5A, dtype=torch.uint8, device=dev)
        n = tokens * heads * d
        ref = (torch.empty(n, dtype=torch.float8_e4m3fn, device=dev).view(tokens, heads, d),
               torch.empty((tokens, heads, d // 32), dtype=torch.uint8, device=dev),
               torch.empty(n, dtype=torch.float8_e4m3fn, device=dev).view(tokens, heads, d),
               torch.empty((tokens // 32, heads, d), dtype=torch.uint8, device=dev))
        lib.projection_mxfp8(*args, heads, d, qr, workspace=wsp, out=ref)
        torch.cuda.synchronize()
        for name, b, s, r in zip(("row codes", "row scales", "col codes", "col scales"), bufs, sizes, ref):
            got = b[:s].cpu().numpy()
            want = r.view(torch.uint8).reshape(-1).cpu().numpy()
            bad = np.flatnonzero(got != want)
            assert len(bad) == 0, f"call {i} {name}: {len(bad)} differ, first {bad[:4].tolist()}"


def test_noalloc_python_binding_and_scratch_limit(lib):
    tokens, heads, d, qr, K = 64, 4, 192, 64, 256
    args = problem(tokens, heads, d, qr, K, seed=5)
    out = lib.projection_mxfp8_noalloc(*args, heads, d, qr)
    ref = lib.projection_mxfp8(*args, heads, d, qr)
    torch.cuda.synchronize()
    for a, b in zip(out, ref):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    # a problem whose workspace exceeds the scratch is refused before any device work
    big = (16384, 128, 192, 64, 7168)
    assert lib._lib.mxgemm_projection_workspace_bytes(big[0], big[1], big[2], big[4]) > \
        lib.MXGEMM_NOALLOC_SCRATCH_BYTES
    bufs = [torch.zeros(16, dtype=torch.uint8, device="cuda:0") for _ in range(4)]
    assert c_abi_noalloc(lib, args, bufs, *big) == lib.MXG_ERR_SCRATCH
