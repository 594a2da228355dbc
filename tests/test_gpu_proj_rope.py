"""The projection page's per-head RoPE and dual-direction MXFP8 quantisation on the GPU
(mxgemm_proj_rope_mxfp8): bit-exact against the oracle on seeded float32 inputs (both
directions' codes and scale bytes), guard bands past every output, and the whole projection
(row-wise scales -> GEMM -> RoPE + quantisation) against the oracle chain."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.codecs import decode, FMT_E4M3

pytestmark = pytest.mark.gpu
E4 = W.FMT_E4M3


@pytest.fixture(scope="module")
def lib():
    import block_scaled_precision_e4m3_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return lib


def inputs(tokens, heads, d, qr, seed):
    rng = np.random.default_rng(seed)
    y = (rng.standard_normal((tokens, heads * d)) * np.exp2(rng.integers(-8, 9, size=(tokens, 1)))).astype(np.float32)
    y[3, :d] = 0.0                                                  # all-zero row blocks of head 0
    y[:32, d:d + 1] = 0.0                                           # an all-zero column block
    cs = torch.from_numpy(rng.uniform(-1, 1, size=(tokens, qr)).astype(np.float32)).to(torch.bfloat16)
    sn = torch.from_numpy(rng.uniform(-1, 1, size=(tokens, qr)).astype(np.float32)).to(torch.bfloat16)
    return y, cs, sn


@pytest.mark.parametrize("tokens,heads,d,qr", [(64, 3, 192, 64), (128, 5, 64, 32), (32, 1, 256, 0), (96, 2, 192, 2)])
def test_rope_quantise_bit_exact(lib, tokens, heads, d, qr):
    print(f"proj rope {tokens}x{heads}x{d} qr={qr}", flush=True)
    y, cs, sn = inputs(tokens, heads, d, qr, seed=tokens + heads + d + qr)
    dev = torch.device("cuda:0")
    g = 4096
    n = tokens * heads * d
    bufs = [torch.full((n + g,), 0xA5, dtype=torch.uint8, device=dev),
            torch.full((n // 32 + g,), 0xA5, dtype=torch.uint8, device=dev),
            torch.full((n + g,), 0xA5, dtype=torch.uint8, device=dev),
            torch.full((n // 32 + g,), 0xA5, dtype=torch.uint8, device=dev)]
    out = (bufs[0][:n].view(torch.float8_e4m3fn).view(tokens, heads, d),
           bufs[1][:n // 32].view(tokens, heads, d // 32),
           bufs[2][:n].view(torch.float8_e4m3fn).view(tokens, heads, d),
           bufs[3][:n // 32].view(tokens // 32, heads, d))
    lib.proj_rope_mxfp8(torch.from_numpy(y).to(dev), cs.to(dev), sn.to(dev), heads, d, qr, out=out)
    torch.cuda.synchronize()
    for b, size in zip(bufs, (n, n // 32, n, n // 32)):
        assert torch.all(b[size:] == 0xA5).item(), "write past an output"
    ref = oracle.proj_rope_mxfp8(y, cs.float().numpy(), sn.float().numpy(), heads, d, qr)
    got = [o.view(torch.uint8).cpu().numpy() for o in out]
    for name, gv, rv in zip(("row codes", "row scales", "col codes", "col scales"), got, ref):
        assert gv.shape == rv.shape, name
        bad = np.argwhere(gv != rv)
        assert len(bad) == 0, f"{name}: {len(bad)} differ, first {bad[:4].tolist()}"


def test_projection_end_to_end(lib):
    # DeepSeek-V3 Q up-projection shape (128 heads x 192, Q_LORA 1536) on 256 tokens:
    # MXFP8 x and w with row-wise scales -> atoms -> GEMM (float32 Y) -> RoPE + dual MXFP8
    tokens, heads, d, qr, q_lora = 256, 128, 192, 64, 1536
    n = heads * d
    rng = np.random.default_rng(31)
    x = rng.standard_normal((tokens, q_lora), dtype=np.float32)
    w = (rng.standard_normal((n, q_lora), dtype=np.float32) / np.float32(np.sqrt(q_lora)))
    xq, _, xe = oracle.mx_quantize(x, 32, E4)
    wq, _, we = oracle.mx_quantize(w, 32, E4)
    x_scale = (xe[0] + 127).astype(np.uint8)
    w_scale = (we[0] + 127).astype(np.uint8)
    theta = rng.uniform(-np.pi, np.pi, size=(tokens, qr // 2))
    cs = torch.from_numpy(np.concatenate([np.cos(theta)] * 2, axis=1).astype(np.float32)).to(torch.bfloat16)
    sn = torch.from_numpy(np.concatenate([np.sin(theta)] * 2, axis=1).astype(np.float32)).to(torch.bfloat16)
    dev = torch.device("cuda:0")
    sfa = lib.sf_from_rowwise(torch.from_numpy(x_scale).to(dev), q_lora, 32)
    sfb = lib.sf_from_rowwise(torch.from_numpy(w_scale).to(dev), q_lora, 32)
    A = torch.from_numpy(np.ascontiguousarray(xq[0])).to(dev)
    B = torch.from_numpy(np.ascontiguousarray(wq[0])).to(dev)
    Y = torch.empty(tokens * n, dtype=torch.float32, device=dev)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    lib.mxgemm_amax(A, B, sfa, sfb, Y, amax, tokens, n, q_lora, 1, 32, E4, E4)
    row, row_s, col, col_s = lib.proj_rope_mxfp8(Y.view(tokens, n), cs.to(dev), sn.to(dev), heads, d, qr)
    torch.cuda.synchronize()
    # oracle chain: the fp64 GEMM, then RoPE in float64 (the reference values)
    sfa_o = oracle.place_scales(x_scale[None], tokens, q_lora, 1, 32)
    sfb_o = oracle.place_scales(w_scale[None], n, q_lora, 1, 32)
    y_ref, s_ref = oracle.gemm_rows(xq, wq, sfa_o, sfb_o, tokens, n, q_lora, 1, 32, E4, E4, 0, np.arange(tokens))
    y3, s3 = y_ref.reshape(tokens, heads, d), s_ref.reshape(tokens, heads, d)
    c64, s64 = cs.double().numpy()[:, None, :], sn.double().numpy()[:, None, :]
    nope, r = d - qr, qr // 2
    z = y3.copy()
    a, b = y3[:, :, nope::2], y3[:, :, nope + 1::2]
    z[:, :, nope:nope + r] = a * c64[:, :, :r] - b * s64[:, :, :r]
    z[:, :, nope + r:] = b * c64[:, :, r:] + a * s64[:, :, r:]
    # bound: the GEMM tolerance carried through the rotation (|cos|, |sin| <= 1), float32 rounding of
    # the rotation, and one E4M3 code step (relative 2^-3, or 2^(e-9) below the normal range)
    sb = s3.copy()
    sb[:, :, nope:] = np.concatenate([s3[:, :, nope::2] + s3[:, :, nope + 1::2]] * 2, axis=2)
    for codes, scales, axis in ((row, row_s, 2), (col, col_s, 0)):
        e = scales.cpu().numpy().astype(np.int64) - 127
        e_full = np.repeat(e, 32, axis=axis)
        deq = decode(codes.view(torch.uint8).cpu().numpy(), FMT_E4M3) * np.exp2(e_full)
        bound = 2.0 ** -3 * np.abs(z) + np.exp2(e_full - 9.0) + 2e-5 * sb + 2.0 ** -22 * np.abs(z) + 1e-30
        worst = float(np.max(np.abs(deq - z) / bound))
        assert worst <= 1.0, f"axis {axis}: max |deq - z| / bound = {worst}"


@pytest.mark.parametrize("tokens", [2048, 8192])   # runs of 4 and of 16 heads per workgroup on 256 CUs
def test_rope_quantise_large_sampled_blocks(lib, tokens):
    heads, d, qr = 128, 192, 64
    print(f"proj rope {tokens} tokens, sampled token blocks", flush=True)
    rng = np.random.default_rng(tokens)
    y = rng.standard_normal((tokens, heads * d), dtype=np.float32)
    y *= np.exp2(rng.integers(-8, 9, size=(tokens, 1))).astype(np.float32)
    cs = torch.from_numpy(rng.uniform(-1, 1, size=(tokens, qr)).astype(np.float32)).to(torch.bfloat16)
    sn = torch.from_numpy(rng.uniform(-1, 1, size=(tokens, qr)).astype(np.float32)).to(torch.bfloat16)
    dev = torch.device("cuda:0")
    out = lib.proj_rope_mxfp8(torch.from_numpy(y).to(dev), cs.to(dev), sn.to(dev), heads, d, qr)
    torch.cuda.synchronize()
    got = [o.view(torch.uint8).cpu().numpy() for o in out]
    cf, sf = cs.float().numpy(), sn.float().numpy()
    for tb in (0, 1, tokens // 64, tokens // 32 - 1):   # blocks of 32 tokens are independent
        s = slice(32 * tb, 32 * tb + 32)
        ref = oracle.proj_rope_mxfp8(y[s], cf[s], sf[s], heads, d, qr)
        assert np.array_equal(got[0][s], ref[0]), f"row codes, block {tb}"
        assert np.array_equal(got[1][s], ref[1]), f"row scales, block {tb}"
        assert np.array_equal(got[2][s], ref[2]), f"col codes, block {tb}"
        assert np.array_equal(got[3][tb:tb + 1], ref[3]), f"col scales, block {tb}"
