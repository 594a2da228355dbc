"""The projection with RoPE and dual-direction MXFP8 fused into the GEMM's epilogue
(mxgemm_gemm_rope_mxfp8, mxgemm_projection_mxfp8).

Its four outputs must equal, bit for bit, the oracle's RoPE + quantisation
(oracle.proj_rope_mxfp8) of the float32 Y that the plain GEMM (mxgemm_amax_ex,
256x256 tiles) computes for the same operands: the accumulation is the same
per output, only the epilogue differs.  The plain GEMM's Y is itself checked
against the fp64 oracle elsewhere, and the unfused RoPE kernel on it in
test_gpu_proj_rope.py.  Also: guard bands past every output, ragged token
tiles, several head sizes and rotary widths, both block sizes and element
formats, the row-wise-scale entry point against the atom one, and the rules.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
E4, E5 = W.FMT_E4M3, W.FMT_E5M2
GUARD = 4096


@pytest.fixture(scope="module")
def lib():
    import block_scaled_precision_e4m3_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return lib


def rope_tables(tokens, qr, seed):
    rng = np.random.default_rng(seed)
    theta = rng.uniform(0, 2 * np.pi, size=(tokens, max(qr // 2, 1)))
    cs = np.concatenate([np.cos(theta), np.cos(theta)], axis=1)[:, :qr]
    sn = np.concatenate([np.sin(theta), np.sin(theta)], axis=1)[:, :qr]
    # distinct second halves, so that the index of the second member is exercised
    cs[:, qr // 2:] *= 0.75
    sn[:, qr // 2:] *= -1.25
    return (torch.from_numpy(cs.astype(np.float32)).to(torch.bfloat16),
            torch.from_numpy(sn.astype(np.float32)).to(torch.bfloat16))


def guarded_outputs(tokens, heads, d):
    dev = torch.device("cuda:0")
    n = tokens * heads * d
    sizes = (n, n // 32, n, n // 32)
    bufs = [torch.full((s + GUARD,), 0xA5, dtype=torch.uint8, device=dev) for s in sizes]
    out = (bufs[0][:n].view(torch.float8_e4m3fn).view(tokens, heads, d),
           bufs[1][:n // 32].view(tokens, heads, d // 32),
           bufs[2][:n].view(torch.float8_e4m3fn).view(tokens, heads, d),
           bufs[3][:n // 32].view(tokens // 32, heads, d))
    return bufs, sizes, out


def check_guards(bufs, sizes):
    for b, s in zip(bufs, sizes):
        assert torch.all(b[s:] == 0xA5).item(), "write past an output"


def plain_y(lib, p, d_):
    """float32 Y of the plain GEMM with 256x256 tiles (the fused kernel's tile)."""
    M, N, K, sf = p["M"], p["N"], p["K"], p["sf"]
    C = torch.empty(M * N, dtype=torch.float32, device="cuda:0")
    am = torch.zeros(4, dtype=torch.float32, device="cuda:0")
    lib.mxgemm_amax_ex(d_["A"], d_["B"], d_["SFA"], d_["SFB"], C, am, M, N, K, 1, sf, p["a_fmt"], p["b_fmt"],
                       lib.MXG_FLAG_TILE_256)
    torch.cuda.synchronize()
    return C.view(M, N).cpu().numpy()


def compare(got, ref):
    for name, g, r in zip(("row codes", "row scales", "col codes", "col scales"), got, ref):
        g = g.view(torch.uint8).cpu().numpy()
        assert g.shape == r.shape, name
        bad = np.argwhere(g != r)
        assert len(bad) == 0, f"{name}: {len(bad)} differ, first {bad[:4].tolist()}"


CASES = [
    # tokens, heads, head_dim, qk_rope, K, sf, a_fmt, b_fmt
    (256, 4, 192, 64, 1536, 32, E4, E4),     # the page's head shape
    (288, 8, 192, 64, 512, 32, E4, E4),      # a ragged token tile (32 rows of the second)
    (512, 2, 128, 64, 384, 32, E4, E4),      # one rotary segment per 128-column wave block
    (256, 3, 256, 32, 256, 32, E4, E4),
    (64, 4, 192, 0, 128, 32, E4, E4),        # no rotary features
    (256, 4, 192, 48, 640, 16, E5, E4),      # sf = 16, E5M2 x E4M3
]


@pytest.mark.parametrize("tokens,heads,d,qr,K,sf,fa,fb", CASES)
def test_fused_equals_rope_quantise_of_the_gemm(lib, tokens, heads, d, qr, K, sf, fa, fb):
    print(f"fused projection {tokens} tokens, {heads}x{d}, qr={qr}, K={K}, sf={sf}", flush=True)
    n = heads * d
    p = W.make_problem(tokens, n, K, 1, sf, fa, fb, seed=tokens + n + K + qr)
    dev = torch.device("cuda:0")
    d_ = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev) for k in ("A", "B", "SFA", "SFB")}
    cs, sn = rope_tables(tokens, qr, seed=qr + 1)
    bufs, sizes, out = guarded_outputs(tokens, heads, d)
    lib.gemm_rope_mxfp8(d_["A"], d_["B"], d_["SFA"], d_["SFB"], cs.to(dev), sn.to(dev), tokens, heads, d, qr, K,
                        sf_vec_size=sf, a_fmt=fa, b_fmt=fb, out=out)
    torch.cuda.synchronize()
    check_guards(bufs, sizes)
    y = plain_y(lib, p, d_)
    ref = oracle.proj_rope_mxfp8(y, cs.float().numpy(), sn.float().numpy(), heads, d, qr)
    compare(out, ref)


def test_fused_wide_exponent_range(lib):
    # token rows scaled by 2^U(-10, 10) before MX quantisation: Y's row blocks span about
    # twenty exponents (row codes at many block scales), and each 32-token column block
    # mixes rows far apart in size (column codes down to subnormal and zero); bit-exact
    # against the oracle's RoPE + quantisation of the plain GEMM's Y
    tokens, heads, d, qr, K = 256, 4, 192, 64, 768
    n = heads * d
    print(f"fused projection, wide exponents: {tokens} tokens, {heads}x{d}, K={K}", flush=True)
    rng = np.random.default_rng(99)
    x = rng.standard_normal((1, tokens, K)) * np.exp2(rng.uniform(-10, 10, size=(1, tokens, 1)))
    w = rng.standard_normal((1, n, K)) / np.sqrt(K)
    xq, xs = W.mx_quantize(x.astype(np.float32), 32, E4)
    wq, ws = W.mx_quantize(w.astype(np.float32), 32, E4)
    p = dict(A=xq, B=wq, SFA=W.pack_sf(xs, tokens, K, 1, 32), SFB=W.pack_sf(ws, n, K, 1, 32),
             M=tokens, N=n, K=K, L=1, sf=32, a_fmt=E4, b_fmt=E4)
    dev = torch.device("cuda:0")
    d_ = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev) for k in ("A", "B", "SFA", "SFB")}
    cs, sn = rope_tables(tokens, qr, seed=5)
    bufs, sizes, out = guarded_outputs(tokens, heads, d)
    lib.gemm_rope_mxfp8(d_["A"], d_["B"], d_["SFA"], d_["SFB"], cs.to(dev), sn.to(dev), tokens, heads, d, qr, K,
                        out=out)
    torch.cuda.synchronize()
    check_guards(bufs, sizes)
    y = plain_y(lib, p, d_)
    rs = out[1].cpu().numpy().astype(int)
    assert rs.max() - rs.min() >= 16, "row scales should span a wide range"
    ref = oracle.proj_rope_mxfp8(y, cs.float().numpy(), sn.float().numpy(), heads, d, qr)
    compare(out, ref)


def rowwise_problem(tokens, n, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((1, tokens, k)).astype(np.float32)
    w = (rng.standard_normal((1, n, k)) / np.sqrt(k)).astype(np.float32)
    xq, xs = W.mx_quantize(x, 32, E4)
    wq, ws = W.mx_quantize(w, 32, E4)
    return xq[0], xs[0], wq[0], ws[0]


@pytest.mark.parametrize("tokens,heads,d,qr,K", [(256, 128, 192, 64, 1536), (96, 4, 192, 64, 160)])
def test_rowwise_entry_equals_atom_entry(lib, tokens, heads, d, qr, K):
    # the page's interface (row-wise x_scale / w_scale) through a caller-given
    # workspace gives bitwise the atom-layout call's outputs
    n = heads * d
    xq, xs, wq, ws = rowwise_problem(tokens, n, K, seed=7)
    dev = torch.device("cuda:0")
    x, w = torch.from_numpy(xq).to(dev), torch.from_numpy(wq).to(dev)
    xst, wst = torch.from_numpy(np.ascontiguousarray(xs)).to(dev), torch.from_numpy(np.ascontiguousarray(ws)).to(dev)
    cs, sn = rope_tables(tokens, qr, seed=3)
    cs, sn = cs.to(dev), sn.to(dev)
    need = lib._lib.mxgemm_projection_workspace_bytes(tokens, heads, d, K)
    wsp = torch.full((need + 256,), 0x5A, dtype=torch.uint8, device=dev)
    bufs, sizes, out = guarded_outputs(tokens, heads, d)
    lib.projection_mxfp8(x, w, xst, wst, cs, sn, heads, d, qr, workspace=wsp[:need], out=out)
    torch.cuda.synchronize()
    check_guards(bufs, sizes)
    assert torch.all(wsp[need:] == 0x5A).item(), "write past the workspace"
    sfa = torch.from_numpy(W.pack_sf(xs[None], tokens, K, 1, 32)).to(dev)
    sfb = torch.from_numpy(W.pack_sf(ws[None], n, K, 1, 32)).to(dev)
    ref = lib.gemm_rope_mxfp8(x, w, sfa, sfb, cs, sn, tokens, heads, d, qr, K)
    torch.cuda.synchronize()
    for a, b in zip(out, ref):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_projection_rules(lib):
    f = lib._lib.mxgemm_gemm_rope_mxfp8
    good = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda:0").data_ptr()
    args = [good] * 10

    def st(tokens, heads, d, qr, K, sf=32, fa=E4, fb=E4):
        return f(*args, tokens, heads, d, qr, K, sf, fa, fb, None)
    assert st(64, 4, 192, 64, 0) == lib.MXG_ERR_SHAPE          # K = 0
    assert st(48, 4, 192, 64, 128) == lib.MXG_ERR_ALIGN        # tokens % 32
    assert st(64, 4, 160, 64, 128) == lib.MXG_ERR_SHAPE        # rotary features cross a 128-column boundary
    assert st(64, 4, 96, 32, 128) == lib.MXG_ERR_SHAPE         # head_dim < 128
    assert st(64, 4, 192, 80, 128) == lib.MXG_ERR_SHAPE        # qk_rope > 64
    assert st(64, 4, 192, 24, 128) == lib.MXG_ERR_SHAPE        # qk_rope % 16
    assert st(64, 3, 160, 0, 128) == lib.MXG_ERR_SHAPE         # N % 128
    assert st(64, 4, 192, 64, 128, sf=64) == lib.MXG_ERR_SFVEC
    assert st(64, 4, 192, 64, 128, fa=2) == lib.MXG_ERR_FMT
