"""Helpers shared by the GPU parity tests: upload, run through the C ABI, compare.

The tolerance is the one stated for this path: per element
|C_gpu - C_ref| <= 1e-5 * sum_k |A_hat||B_hat| + 1e-30, and a relative
Amax error <= 1e-5.
"""

import numpy as np

TOL_REL = 1e-5
TOL_ABS = 1e-30
AMAX_REL = 1e-5


def to_device(problem, pad_c=0, c_fill=float("nan")):
    """Copy a workloads problem to cuda:0; returns a dict of device tensors (C with optional guard band)."""
    import torch
    dev = torch.device("cuda:0")
    M, N, L = problem["M"], problem["N"], problem["L"]
    d = dict(
        A=torch.from_numpy(np.ascontiguousarray(problem["A"])).to(dev),
        B=torch.from_numpy(np.ascontiguousarray(problem["B"])).to(dev),
        SFA=torch.from_numpy(np.ascontiguousarray(problem["SFA"])).to(dev),
        SFB=torch.from_numpy(np.ascontiguousarray(problem["SFB"])).to(dev),
    )
    c_full = torch.full((L * M * N + 2 * pad_c,), c_fill, dtype=torch.float32, device=dev)
    d["C_full"] = c_full
    d["C"] = c_full[pad_c:pad_c + L * M * N]
    d["Amax"] = torch.full((4,), -1.0, dtype=torch.float32, device=dev)
    return d


def run(lib, problem, d, flags=0, stream=None):
    """One call of mxgemm_amax_ex through the C ABI on the device buffers."""
    p = problem
    lib.mxgemm_amax_ex(d["A"], d["B"], d["SFA"], d["SFB"], d["C"], d["Amax"], p["M"], p["N"], p["K"], p["L"],
                       p["sf"], p["a_fmt"], p["b_fmt"], flags, stream)


def fetch(problem, d):
    import torch
    torch.cuda.synchronize()
    c = d["C"].cpu().numpy().reshape(problem["L"], problem["M"], problem["N"])
    amax = float(d["Amax"][0].item())
    return c, amax


def check_c(c_gpu, c_ref, s_ref, where=""):
    """Assert the per-element tolerance; returns the largest |diff| / bound."""
    c_gpu = np.asarray(c_gpu, dtype=np.float64)
    bound = TOL_REL * s_ref + TOL_ABS
    diff = np.abs(c_gpu - c_ref)
    bad = ~(diff <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{where}: {int(bad.sum())} of {bad.size} outside tolerance; first "
                             f"{idx.tolist()} gpu={c_gpu[tuple(idx.T)]} ref={c_ref[tuple(idx.T)]}")
    return float(np.max(diff / bound)) if diff.size else 0.0


def check_amax(amax_gpu, amax_ref, where=""):
    assert abs(amax_gpu - amax_ref) <= AMAX_REL * abs(amax_ref), f"{where}: amax gpu {amax_gpu} ref {amax_ref}"


def amax_bits_of(c_gpu):
    """max |C| of the GPU output, as its float32 bit pattern (NaN-propagating like the kernel)."""
    bits = np.asarray(c_gpu, dtype=np.float32).view(np.uint32) & np.uint32(0x7FFFFFFF)
    return int(bits.max()) if bits.size else 0


def float_bits(x):
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])
