"""Block-scaled FP8 GEMM with a fused global-amax epilogue on MI355X (gfx950).

Thin Python binding over the C ABI of ``libmxgemm.so`` (declared in
``include/mxgemm.h``).  Every step of the computation runs in the library's
HIP kernels; this module only marshals arguments (PyTorch supplies device
memory and streams).  It fails loudly when the library has not been built.

Low-level functions carry the C names and arguments:
``mxgemm_amax``, ``mxgemm_amax_ex``, ``mxgemm_amax_reset``,
``mxgemm_check_support``, ``mxgemm_sf_bytes``, ``mxgemm_launch_config``,
``mxgemm_strerror``.  Buffers may be torch tensors (their data pointer is
passed) or integer device addresses.

``gemm_amax`` mirrors the page's high-level wrapper ("GEMM + Amax (SM100)",
section "High-level wrapper"): it takes A (M, K, L) / B (N, K, L) k-major
tensors (or (L, M, K)-contiguous storage viewed that way), SF tensors in the
logical atom view or the physical shape, allocates C (M, N, L) n-major and
Amax (1, 1, 1) when not given, and returns (c, amax).
"""

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libmxgemm.so")

MXG_FMT_E4M3 = 0
MXG_FMT_E5M2 = 1
MXG_FMT_E2M1 = 2
MXG_FLAG_AMAX_ACCUMULATE = 1
MXG_FLAG_FP8_MFMA = 2
MXG_FLAG_TILE_128 = 4
MXG_FLAG_TILE_256 = 8
MXG_FLAG_C_BF16 = 32
MXG_FLAG_C_F16 = 64
MXG_FLAG_C_MMAJOR = 128
MXG_FLAG_A_MMAJOR = 256
MXG_FLAG_B_NMAJOR = 512

MXG_OK = 0
MXG_ERR_NULL = -1
MXG_ERR_SHAPE = -2
MXG_ERR_ALIGN = -3
MXG_ERR_SFVEC = -4
MXG_ERR_FMT = -5
MXG_ERR_DEVICE = -6
MXG_ERR_LAUNCH = -7
MXG_ERR_FLAGS = -8
MXG_ERR_SCRATCH = -9
MXGEMM_NOALLOC_SCRATCH_BYTES = 8 << 20  # fixed per-device scratch of the _noalloc entry

EXPORTED = ("mxgemm_amax", "mxgemm_amax_ex", "mxgemm_amax_reset", "mxgemm_check_support",
            "mxgemm_sf_bytes", "mxgemm_launch_config", "mxgemm_strerror", "mxgemm_mx_quantize",
            "mxgemm_sf_rowwise_to_atoms", "mxgemm_plan_init", "mxgemm_plan_execute", "mxgemm_codes_to_kmajor",
            "mxgemm_proj_rope_mxfp8", "mxgemm_gemm_rope_mxfp8", "mxgemm_projection_workspace_bytes",
            "mxgemm_projection_mxfp8", "mxgemm_projection_mxfp8_noalloc")


class MxgemmError(Exception):
    def __init__(self, status, msg):
        super().__init__(f"mxgemm status {status}: {msg}")
        self.status = status


class MxgemmValueError(MxgemmError, ValueError):
    pass


class MxgemmRuntimeError(MxgemmError, RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first with "
            "`python -m block_scaled_precision_e4m3_amd._build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, ci, cu = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint
    gemm_args = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ci, ci, ci]
    lib.mxgemm_amax.argtypes = gemm_args + [vp]
    lib.mxgemm_amax.restype = ci
    lib.mxgemm_amax_ex.argtypes = gemm_args + [cu, vp]
    lib.mxgemm_amax_ex.restype = ci
    lib.mxgemm_amax_reset.argtypes = [vp, vp]
    lib.mxgemm_amax_reset.restype = ci
    lib.mxgemm_check_support.argtypes = [i64, i64, i64, i64, ci, ci, ci]
    lib.mxgemm_check_support.restype = ci
    lib.mxgemm_sf_bytes.argtypes = [i64, i64, i64, ci]
    lib.mxgemm_sf_bytes.restype = ctypes.c_size_t
    lib.mxgemm_launch_config.argtypes = [i64, i64, i64, i64, ci, ctypes.POINTER(ci), ctypes.POINTER(ci),
                                         ctypes.POINTER(i64)]
    lib.mxgemm_launch_config.restype = ci
    lib.mxgemm_strerror.argtypes = [ci]
    lib.mxgemm_strerror.restype = ctypes.c_char_p
    lib.mxgemm_mx_quantize.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
    lib.mxgemm_mx_quantize.restype = ci
    lib.mxgemm_sf_rowwise_to_atoms.argtypes = [vp, vp, i64, i64, i64, ci, vp]
    lib.mxgemm_sf_rowwise_to_atoms.restype = ci
    lib.mxgemm_plan_init.argtypes = [vp, i64, i64, i64, i64, ci, ci, ci, cu]
    lib.mxgemm_plan_init.restype = ci
    lib.mxgemm_plan_execute.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mxgemm_plan_execute.restype = ci
    lib.mxgemm_codes_to_kmajor.argtypes = [vp, vp, i64, i64, i64, vp]
    lib.mxgemm_codes_to_kmajor.restype = ci
    lib.mxgemm_proj_rope_mxfp8.argtypes = [vp] * 7 + [i64] * 4 + [vp]
    lib.mxgemm_proj_rope_mxfp8.restype = ci
    lib.mxgemm_gemm_rope_mxfp8.argtypes = [vp] * 10 + [i64] * 5 + [ci, ci, ci, vp]
    lib.mxgemm_gemm_rope_mxfp8.restype = ci
    lib.mxgemm_projection_workspace_bytes.argtypes = [i64] * 4
    lib.mxgemm_projection_workspace_bytes.restype = ctypes.c_size_t
    lib.mxgemm_projection_mxfp8.argtypes = [vp] * 10 + [i64] * 5 + [vp, ctypes.c_size_t, vp]
    lib.mxgemm_projection_mxfp8.restype = ci
    lib.mxgemm_projection_mxfp8_noalloc.argtypes = [vp] * 10 + [i64] * 5 + [vp]
    lib.mxgemm_projection_mxfp8_noalloc.restype = ci
    return lib


_lib = _load()


def _raise(status):
    msg = _lib.mxgemm_strerror(status).decode()
    if status in (MXG_ERR_DEVICE, MXG_ERR_LAUNCH):
        raise MxgemmRuntimeError(status, msg)
    raise MxgemmValueError(status, msg)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def mxgemm_strerror(status):
    return _lib.mxgemm_strerror(int(status)).decode()


def mxgemm_check_support(M, N, K, L, sf_vec_size, a_fmt, b_fmt):
    """Status code (0 = supported) for these sizes and formats; host-only."""
    return _lib.mxgemm_check_support(M, N, K, L, sf_vec_size, a_fmt, b_fmt)


def mxgemm_sf_bytes(MN, K, L, sf_vec_size):
    return _lib.mxgemm_sf_bytes(MN, K, L, sf_vec_size)


def mxgemm_launch_config(M, N, K, L, sf_vec_size, with_grid=True):
    """(tile_m, tile_n, grid) the library would use; grid is None unless with_grid (queries the device)."""
    tm, tn, g = ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
    st = _lib.mxgemm_launch_config(M, N, K, L, sf_vec_size, ctypes.byref(tm), ctypes.byref(tn),
                                   ctypes.byref(g) if with_grid else None)
    if st != MXG_OK:
        _raise(st)
    return tm.value, tn.value, (g.value if with_grid else None)


def mxgemm_amax_ex(A, B, SFA, SFB, C, Amax, M, N, K, L, sf_vec_size, a_fmt, b_fmt, flags=0, stream=None):
    """C-ABI mxgemm_amax_ex on torch tensors or raw device addresses; raises on a nonzero status."""
    st = _lib.mxgemm_amax_ex(_ptr(A), _ptr(B), _ptr(SFA), _ptr(SFB), _ptr(C), _ptr(Amax),
                             M, N, K, L, sf_vec_size, a_fmt, b_fmt, flags, _stream(stream))
    if st != MXG_OK:
        _raise(st)


def mxgemm_amax(A, B, SFA, SFB, C, Amax, M, N, K, L, sf_vec_size, a_fmt, b_fmt, stream=None):
    """C-ABI mxgemm_amax on torch tensors or raw device addresses; raises on a nonzero status."""
    st = _lib.mxgemm_amax(_ptr(A), _ptr(B), _ptr(SFA), _ptr(SFB), _ptr(C), _ptr(Amax),
                          M, N, K, L, sf_vec_size, a_fmt, b_fmt, _stream(stream))
    if st != MXG_OK:
        _raise(st)


def mxgemm_amax_reset(Amax, stream=None):
    st = _lib.mxgemm_amax_reset(_ptr(Amax), _stream(stream))
    if st != MXG_OK:
        _raise(st)


# --- high-level wrapper ---------------------------------------------------------

def _fmt_of(t):
    import torch
    if t.dtype == torch.float8_e4m3fn:
        return MXG_FMT_E4M3
    if t.dtype == torch.float8_e5m2:
        return MXG_FMT_E5M2
    raise MxgemmValueError(MXG_ERR_FMT, f"A/B dtype must be float8_e4m3fn or float8_e5m2, got {t.dtype}")


def _as_lrk(t, name):
    """Return (storage tensor, rows, K, L, m_major) from a (rows, K, L) view or 2-D.

    k-major views (strides (K, 1, rows*K)) come back as (L, rows, K) storage; m-major ones
    (strides (1, rows, rows*K), the pages' m-major A / n-major B) as (L, K, rows) storage with
    m_major True, which the GEMM reads as it is (MXG_FLAG_A_MMAJOR / MXG_FLAG_B_NMAJOR)."""
    import torch
    if t.dim() == 2:
        t = t.unsqueeze(2)
    if t.dim() != 3:
        raise MxgemmValueError(MXG_ERR_SHAPE, f"{name} must be (rows, K) or (rows, K, L)")
    rows, k, l = t.shape
    base = t.permute(2, 0, 1)
    if base.is_contiguous():
        return base, rows, k, l, False
    mmajor = t.permute(2, 1, 0)
    if mmajor.is_contiguous() and t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return mmajor, rows, k, l, True
    raise MxgemmValueError(MXG_ERR_ALIGN, f"{name} must be k-major (strides (K, 1, rows*K)) or, for FP8 codes, "
                                          f"m-major (strides (1, rows, rows*K)), batch outermost")


def proj_rope_mxfp8(y, cos, sin, num_heads, head_dim=192, qk_rope=64, stream=None, out=None):
    """C-ABI mxgemm_proj_rope_mxfp8 on torch tensors: y (tokens, num_heads * head_dim) float32, cos / sin
    (tokens, qk_rope) bfloat16.  Returns (out_fp8_row, out_scales_row, out_fp8_col, out_scales_col) as the
    projection page's wrapper does: codes (tokens, H, D) float8_e4m3fn, scales uint8 (tokens, H, D/32) and
    (tokens/32, H, D); `out` may hold those four tensors preallocated."""
    import torch
    tokens = y.shape[0]
    if out is None:
        dev = y.device
        out = (torch.empty((tokens, num_heads, head_dim), dtype=torch.float8_e4m3fn, device=dev),
               torch.empty((tokens, num_heads, head_dim // 32), dtype=torch.uint8, device=dev),
               torch.empty((tokens, num_heads, head_dim), dtype=torch.float8_e4m3fn, device=dev),
               torch.empty((tokens // 32, num_heads, head_dim), dtype=torch.uint8, device=dev))
    for t, name in ((y, "y"), (cos, "cos"), (sin, "sin")) + tuple(zip(out, ("row", "row scales", "col",
                                                                         "col scales"))):
        if not t.is_contiguous():
            raise MxgemmValueError(MXG_ERR_ALIGN, f"{name} must be contiguous")
    if y.dtype != torch.float32 or cos.dtype != torch.bfloat16 or sin.dtype != torch.bfloat16:
        raise MxgemmValueError(MXG_ERR_FMT, "y must be float32, cos and sin bfloat16")
    st = _lib.mxgemm_proj_rope_mxfp8(_ptr(y), _ptr(cos), _ptr(sin), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]),
                                     _ptr(out[3]), tokens, num_heads, head_dim, qk_rope, _stream(stream))
    if st != MXG_OK:
        _raise(st)
    return out


def _proj_outputs(tokens, num_heads, head_dim, dev, out):
    import torch
    if out is None:
        out = (torch.empty((tokens, num_heads, head_dim), dtype=torch.float8_e4m3fn, device=dev),
               torch.empty((tokens, num_heads, head_dim // 32), dtype=torch.uint8, device=dev),
               torch.empty((tokens, num_heads, head_dim), dtype=torch.float8_e4m3fn, device=dev),
               torch.empty((tokens // 32, num_heads, head_dim), dtype=torch.uint8, device=dev))
    for t, name in zip(out, ("row", "row scales", "col", "col scales")):
        if not t.is_contiguous():
            raise MxgemmValueError(MXG_ERR_ALIGN, f"{name} must be contiguous")
    return out


def gemm_rope_mxfp8(A, B, SFA, SFB, cos, sin, tokens, num_heads, head_dim, qk_rope, K, sf_vec_size=32,
                    a_fmt=MXG_FMT_E4M3, b_fmt=MXG_FMT_E4M3, stream=None, out=None):
    """C-ABI mxgemm_gemm_rope_mxfp8: the projection GEMM with RoPE and dual-direction MXFP8 fused into its
    epilogue, on k-major codes A (tokens, K) / B (num_heads * head_dim, K) and atom-layout scales.  Returns
    (out_fp8_row, out_scales_row, out_fp8_col, out_scales_col) shaped as proj_rope_mxfp8's."""
    out = _proj_outputs(tokens, num_heads, head_dim, A.device, out)
    st = _lib.mxgemm_gemm_rope_mxfp8(_ptr(A), _ptr(B), _ptr(SFA), _ptr(SFB), _ptr(cos), _ptr(sin), _ptr(out[0]),
                                     _ptr(out[1]), _ptr(out[2]), _ptr(out[3]), tokens, num_heads, head_dim, qk_rope,
                                     K, sf_vec_size, a_fmt, b_fmt, _stream(stream))
    if st != MXG_OK:
        _raise(st)
    return out


def projection_mxfp8(x, w, x_scale, w_scale, cos, sin, num_heads, head_dim=192, qk_rope=64, workspace=None,
                     stream=None, out=None):
    """C-ABI mxgemm_projection_mxfp8, the projection page's MXFP8-input path: x (tokens, K) and w
    (num_heads * head_dim, K) E4M3 codes, row-wise E8M0 scales x_scale (tokens, ceil(K/32)) and w_scale
    (num_heads * head_dim, ceil(K/32)), bf16 cos / sin (tokens, qk_rope).  Allocates the workspace when
    not given.  Returns the four outputs as proj_rope_mxfp8 does."""
    import torch
    tokens, k = x.shape
    need = _lib.mxgemm_projection_workspace_bytes(tokens, num_heads, head_dim, k)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    out = _proj_outputs(tokens, num_heads, head_dim, x.device, out)
    st = _lib.mxgemm_projection_mxfp8(_ptr(x), _ptr(w), _ptr(x_scale), _ptr(w_scale), _ptr(cos), _ptr(sin),
                                      _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(out[3]), tokens, num_heads,
                                      head_dim, qk_rope, k, _ptr(workspace), workspace.numel(), _stream(stream))
    if st != MXG_OK:
        _raise(st)
    return out


def projection_mxfp8_noalloc(x, w, x_scale, w_scale, cos, sin, num_heads, head_dim=192, qk_rope=64,
                             stream=None, out=None):
    """C-ABI mxgemm_projection_mxfp8_noalloc: projection_mxfp8 with the workspace taken from the library's
    fixed per-device scratch array (nothing is allocated; `out` must then be given by a caller that cannot
    allocate either).  Calls that overlap on one device race."""
    tokens, k = x.shape
    out = _proj_outputs(tokens, num_heads, head_dim, x.device, out)
    st = _lib.mxgemm_projection_mxfp8_noalloc(_ptr(x), _ptr(w), _ptr(x_scale), _ptr(w_scale), _ptr(cos),
                                              _ptr(sin), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(out[3]),
                                              tokens, num_heads, head_dim, qk_rope, k, _stream(stream))
    if st != MXG_OK:
        _raise(st)
    return out


def codes_to_kmajor(src, dst, MN, K, L, stream=None):
    """C-ABI mxgemm_codes_to_kmajor: (L, K, MN) codes into (L, MN, K); raises on a nonzero status."""
    st = _lib.mxgemm_codes_to_kmajor(_ptr(src), _ptr(dst), MN, K, L, _stream(stream))
    if st != MXG_OK:
        _raise(st)


def _sf_phys(t, mn, k, l, sf):
    """Accept the logical SF view (32, 4, MNb, 4, Kg, L) or the physical (L, MNb, Kg, 32, 4, 4) / flat bytes."""
    import torch
    mnb, kg = -(-mn // 128), -(-k // (4 * sf))
    logical = (32, 4, mnb, 4, kg, l)
    if tuple(t.shape) == logical and t.dim() == 6:
        t = t.permute(5, 2, 4, 0, 1, 3)
    if not t.is_contiguous():
        raise MxgemmValueError(MXG_ERR_ALIGN, "SF tensor must be the physical buffer or its logical view")
    if t.dtype != torch.uint8:
        t = t.view(torch.uint8)
    if t.numel() != 512 * l * mnb * kg:
        raise MxgemmValueError(MXG_ERR_SHAPE, f"SF tensor has {t.numel()} bytes, expected {512 * l * mnb * kg}")
    return t


def gemm_amax(a, b, sfa, sfb, c=None, amax=None, sf_vec_size=32, stream=None, accumulate=False, fp8_mfma=False,
              c_dtype=None, c_major="n"):
    """(c, amax) = block-scaled GEMM + amax of torch FP8 tensors; see the module docstring.

    C is float32 by default; c_dtype (or a preallocated c) of torch.bfloat16 / torch.float16
    stores the accumulators rounded to nearest even (amax still from the float32 values).
    c_major: "n" (C strides (N, 1, M*N), the default) or "m" (strides (1, M, M*N), float32),
    as the pages' wrapper argument of that name."""
    import torch
    a_base, m, k, l, a_mm = _as_lrk(a, "A")
    b_base, n, kb, lb, b_mm = _as_lrk(b, "B")
    if kb != k or lb != l:
        raise MxgemmValueError(MXG_ERR_SHAPE, "A and B disagree on K or L")
    fa, fb = _fmt_of(a), _fmt_of(b)
    sfa_p = _sf_phys(sfa, m, k, l, sf_vec_size)
    sfb_p = _sf_phys(sfb, n, k, l, sf_vec_size)
    if c_major not in ("n", "m"):
        raise MxgemmValueError(MXG_ERR_FLAGS, f"c_major must be 'n' or 'm', got {c_major!r}")
    if c_major == "m":
        if c is None:
            c = torch.empty((l, n, m), dtype=c_dtype or torch.float32, device=a.device).permute(2, 1, 0)
        c_base = c.permute(2, 1, 0) if c.dim() == 3 else c.t().unsqueeze(0)
        c_flag = MXG_FLAG_C_MMAJOR if c.dtype == torch.float32 else None
        if c_flag is None or not c_base.is_contiguous():
            raise MxgemmValueError(MXG_ERR_ALIGN, "m-major C must be float32 (M, N, L) with strides (1, M, M*N)")
    else:
        if c is None:
            c = torch.empty((l, m, n), dtype=c_dtype or torch.float32, device=a.device).permute(1, 2, 0)
        c_base = c.permute(2, 0, 1) if c.dim() == 3 else c.unsqueeze(0)
        c_flag = {torch.float32: 0, torch.bfloat16: MXG_FLAG_C_BF16, torch.float16: MXG_FLAG_C_F16}.get(c.dtype)
        if c_flag is None or not c_base.is_contiguous():
            raise MxgemmValueError(MXG_ERR_ALIGN, "C must be float32, bfloat16 or float16, n-major (M, N, L) with "
                                                  "strides (N, 1, M*N)")
    if amax is None:
        amax = torch.zeros((1, 1, 1), dtype=torch.float32, device=a.device)
    flags = (MXG_FLAG_AMAX_ACCUMULATE if accumulate else 0) | (MXG_FLAG_FP8_MFMA if fp8_mfma else 0) | c_flag | \
        (MXG_FLAG_A_MMAJOR if a_mm else 0) | (MXG_FLAG_B_NMAJOR if b_mm else 0)
    mxgemm_amax_ex(a_base, b_base, sfa_p, sfb_p, c_base, amax, m, n, k, l, sf_vec_size, fa, fb, flags, stream)
    return c, amax


def mxgemm_mx_quantize(X, Q, SF, MN, K, L, sf_vec_size, fmt, stream=None):
    """C-ABI mxgemm_mx_quantize on torch tensors or raw device addresses; raises on a nonzero status."""
    st = _lib.mxgemm_mx_quantize(_ptr(X), _ptr(Q), _ptr(SF), MN, K, L, sf_vec_size, fmt, _stream(stream))
    if st != MXG_OK:
        _raise(st)


class Plan:
    """A validated, configured GEMM + amax launch (C-ABI mxgemm_plan): the pages' class API
    (check_support -> compile -> execute), with the per-call host work reduced to pointer checks.

    plan = Plan(M, N, K, L, sf_vec_size, a_fmt, b_fmt, flags); plan(A, B, SFA, SFB, C, Amax, stream)
    """

    class _C(ctypes.Structure):
        _fields_ = [("opaque", ctypes.c_uint64 * 32)]

    def __init__(self, M, N, K, L, sf_vec_size, a_fmt, b_fmt, flags=0):
        self._plan = Plan._C()
        self._ref = ctypes.byref(self._plan)
        st = _lib.mxgemm_plan_init(self._ref, M, N, K, L, sf_vec_size, a_fmt, b_fmt, flags)
        if st != MXG_OK:
            _raise(st)

    def __call__(self, A, B, SFA, SFB, C, Amax, stream=None):
        st = _lib.mxgemm_plan_execute(self._ref, _ptr(A), _ptr(B), _ptr(SFA), _ptr(SFB), _ptr(C), _ptr(Amax),
                                      _stream(stream))
        if st != MXG_OK:
            _raise(st)


def mxgemm_sf_rowwise_to_atoms(rowwise, SF, MN, K, L, sf_vec_size, stream=None):
    """C-ABI mxgemm_sf_rowwise_to_atoms on torch tensors or raw device addresses; raises on a nonzero status."""
    st = _lib.mxgemm_sf_rowwise_to_atoms(_ptr(rowwise), _ptr(SF), MN, K, L, sf_vec_size, _stream(stream))
    if st != MXG_OK:
        _raise(st)


def sf_from_rowwise(rowwise, k, sf_vec_size=32, sf=None, stream=None):
    """Atom-layout scales (L, ceil(MN/128), ceil(K/(4 sf)), 32, 4, 4) uint8 from a contiguous row-wise
    uint8 CUDA tensor (MN, ceil(K/sf)) or (L, MN, ceil(K/sf)) of E8M0 bytes (e.g. the pages' x_scale)."""
    import torch
    if rowwise.element_size() != 1 or not rowwise.is_contiguous() or rowwise.dim() not in (2, 3):
        raise MxgemmValueError(MXG_ERR_SHAPE, "row-wise scales must be a contiguous one-byte (MN, Kb) or "
                                              "(L, MN, Kb) tensor")
    l, mn, kb = (1,) + tuple(rowwise.shape) if rowwise.dim() == 2 else tuple(rowwise.shape)
    if kb != -(-k // sf_vec_size):
        raise MxgemmValueError(MXG_ERR_SHAPE, f"row-wise scales have {kb} blocks per row, K={k} needs "
                                              f"{-(-k // sf_vec_size)}")
    shape = (l, -(-mn // 128), -(-k // (4 * sf_vec_size)), 32, 4, 4)
    if sf is None:
        sf = torch.empty(shape, dtype=torch.uint8, device=rowwise.device)
    if sf.numel() != 512 * shape[0] * shape[1] * shape[2] or not sf.is_contiguous():
        raise MxgemmValueError(MXG_ERR_SHAPE, "sf must be a contiguous buffer of the atom layout's size")
    mxgemm_sf_rowwise_to_atoms(rowwise, sf, mn, k, l, sf_vec_size, stream)
    return sf


def mx_quantize(x, sf_vec_size=32, fmt=MXG_FMT_E4M3, q=None, sf=None, stream=None):
    """MX-quantise a contiguous float32 CUDA tensor x of shape (MN, K) or (L, MN, K).

    Returns (q, sf): q uint8 codes of x's shape (view it as torch.float8_e4m3fn /
    float8_e5m2 for gemm_amax) and sf, the physical atom-layout scale buffer
    (L, ceil(MN/128), ceil(K/(4 sf)), 32, 4, 4) uint8, which gemm_amax accepts
    as SFA / SFB.  Preallocated q / sf are used when given.
    """
    import torch
    if x.dtype != torch.float32 or not x.is_contiguous() or x.dim() not in (2, 3):
        raise MxgemmValueError(MXG_ERR_ALIGN, "x must be a contiguous float32 (MN, K) or (L, MN, K) tensor")
    l, mn, k = (1,) + tuple(x.shape) if x.dim() == 2 else tuple(x.shape)
    shape = (l, -(-mn // 128), -(-k // (4 * sf_vec_size)), 32, 4, 4)
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty(shape, dtype=torch.uint8, device=x.device)
    if q.numel() != x.numel() or not q.is_contiguous() or q.element_size() != 1:
        raise MxgemmValueError(MXG_ERR_SHAPE, "q must be a contiguous one-byte tensor with x's element count")
    if sf.numel() != 512 * shape[0] * shape[1] * shape[2] or not sf.is_contiguous():
        raise MxgemmValueError(MXG_ERR_SHAPE, f"sf must be a contiguous buffer of {512 * shape[0] * shape[1] * shape[2]} bytes")
    mxgemm_mx_quantize(x, q, sf, mn, k, l, sf_vec_size, fmt, stream)
    return q, sf


__all__ = [
    "mxgemm_amax", "mxgemm_amax_ex", "mxgemm_amax_reset", "mxgemm_check_support", "mxgemm_sf_bytes",
    "mxgemm_launch_config", "mxgemm_strerror", "gemm_amax", "LIB_PATH", "EXPORTED",
    "mxgemm_mx_quantize", "mx_quantize", "mxgemm_sf_rowwise_to_atoms", "sf_from_rowwise", "Plan",
    "MXG_FMT_E4M3", "MXG_FMT_E5M2", "MXG_FMT_E2M1", "MXG_FLAG_AMAX_ACCUMULATE", "MXG_FLAG_FP8_MFMA", "MXG_FLAG_TILE_128",
    "MXG_FLAG_TILE_256", "MXG_FLAG_C_BF16", "MXG_FLAG_C_F16", "MXG_FLAG_C_MMAJOR", "MXG_FLAG_A_MMAJOR",
    "MXG_FLAG_B_NMAJOR", "codes_to_kmajor",
    "proj_rope_mxfp8", "gemm_rope_mxfp8", "projection_mxfp8", "projection_mxfp8_noalloc", "MxgemmError",
    "MxgemmValueError",
    "MxgemmRuntimeError",
]
