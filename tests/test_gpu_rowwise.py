"""Row-wise E8M0 scales (the projection page's x_scale / w_scale form) into the
atom layout: bit-exact against the oracle's placement, and end to end, a GEMM
fed with repacked row-wise scales equals the GEMM on the oracle's atoms."""

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

E4 = oracle.FMT_E4M3


@pytest.fixture(scope="module")
def lib():
    import block_scaled_precision_e4m3_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return lib


@pytest.mark.parametrize("sf", [16, 32])
@pytest.mark.parametrize("shape", [(1, 128, 128), (1, 300, 176), (3, 130, 48), (2, 1, 16), (1, 520, 1040)])
def test_repack_matches_oracle_placement(lib, shape, sf):
    l, mn, k = shape
    kb = -(-k // sf)
    rw = np.random.default_rng(mn + k + sf).integers(0, 256, size=(l, mn, kb), dtype=np.uint8)
    print(f"repack {shape} sf={sf}", flush=True)
    got = lib.sf_from_rowwise(torch.from_numpy(rw).cuda(), k, sf)
    torch.cuda.synchronize()
    want = oracle.place_scales(rw, mn, k, l, sf)
    assert np.array_equal(got.cpu().numpy().reshape(-1), want)


def test_rowwise_projection_gemm_end_to_end(lib):
    # the projection page's MXFP8-input GEMM at a reduced token count: x (tokens, Q_LORA) and
    # w (NUM_HEADS * HEAD_DIM, Q_LORA) quantised with row-wise scales, repacked, multiplied
    tokens, heads, head_dim, q_lora = 256, 128, 192, 1536
    n = heads * head_dim
    rng = np.random.default_rng(12)
    x = rng.standard_normal((tokens, q_lora), dtype=np.float32)
    w = (rng.standard_normal((n, q_lora), dtype=np.float32) / np.float32(np.sqrt(q_lora)))
    xq, _, xe = oracle.mx_quantize(x, 32, E4)
    wq, _, we = oracle.mx_quantize(w, 32, E4)
    x_scale = (xe[0] + 127).astype(np.uint8)          # (tokens, Q_LORA / 32), row-wise
    w_scale = (we[0] + 127).astype(np.uint8)          # (n, Q_LORA / 32)
    print("row-wise projection GEMM", flush=True)
    sfa = lib.sf_from_rowwise(torch.from_numpy(x_scale).cuda(), q_lora, 32)
    sfb = lib.sf_from_rowwise(torch.from_numpy(w_scale).cuda(), q_lora, 32)
    A = torch.from_numpy(np.ascontiguousarray(xq[0])).cuda()
    B = torch.from_numpy(np.ascontiguousarray(wq[0])).cuda()
    c1 = torch.empty(tokens * n, dtype=torch.float32, device="cuda")
    c2 = torch.empty_like(c1)
    a1 = torch.zeros(1, dtype=torch.float32, device="cuda")
    a2 = torch.zeros_like(a1)
    lib.mxgemm_amax(A, B, sfa, sfb, c1, a1, tokens, n, q_lora, 1, 32, E4, E4)
    sfa_o = torch.from_numpy(oracle.place_scales(x_scale[None], tokens, q_lora, 1, 32)).cuda()
    sfb_o = torch.from_numpy(oracle.place_scales(w_scale[None], n, q_lora, 1, 32)).cuda()
    lib.mxgemm_amax(A, B, sfa_o, sfb_o, c2, a2, tokens, n, q_lora, 1, 32, E4, E4)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(a1, a2)
    rows = np.array([0, 77, tokens - 1])
    cref, sref = oracle.gemm_rows(xq, wq, sfa_o.cpu().numpy(), sfb_o.cpu().numpy(), tokens, n, q_lora, 1, 32,
                                  E4, E4, 0, rows)
    got = c1.view(tokens, n)[rows].double().cpu().numpy()
    assert np.all(np.abs(got - cref) <= 1e-5 * sref + 1e-30)
