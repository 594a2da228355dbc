"""CPU checks of the C ABI: the library loads, exports every function the
header declares, and its host-side validation returns the documented status
codes before touching a device (no kernel is launched here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxgemm.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))


@pytest.fixture(scope="module")
def lib():
    import __graft_entry__
    if not os.path.exists(os.path.join(ROOT, "block_scaled_precision_e4m3_amd", "libmxgemm.so")):
        __graft_entry__.build()
    import block_scaled_precision_e4m3_amd as lib
    return lib


def declared_functions(headers=(HEADER,), prefix="mxgemm_"):
    names = set()
    for h in headers:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(" + prefix + r"\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_expected_set(lib):
    assert declared_functions() == sorted(lib.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    # every function of every header under include/ (the GEMM library and its probes)
    cdll = ctypes.CDLL(lib.LIB_PATH)
    names = declared_functions(HEADERS, prefix="mx(?:gemm|probe)_")
    assert any(n.startswith("mxprobe_") for n in names)
    for name in names:
        assert hasattr(cdll, name), name


def test_status_codes_match_header(lib):
    text = open(HEADER).read()
    for name, val in re.findall(r"\b(MXG_\w+)\s*=\s*(-?\d+)", text):
        assert getattr(lib, name) == int(val), name
    m = re.search(r"#define MXGEMM_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and lib.MXGEMM_NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))


def test_check_support(lib):
    ok = lib.mxgemm_check_support
    assert ok(256, 256, 256, 1, 32, 0, 0) == lib.MXG_OK
    assert ok(4000, 7168, 2048, 1, 16, 1, 0) == lib.MXG_OK
    assert ok(0, 0, 0, 0, 32, 0, 0) == lib.MXG_OK
    assert ok(-1, 256, 256, 1, 32, 0, 0) == lib.MXG_ERR_SHAPE
    assert ok(256, 256, 256, 1, 8, 0, 0) == lib.MXG_ERR_SFVEC
    assert ok(256, 256, 256, 1, 16, 2, 2) == lib.MXG_OK      # packed FP4 at sf = 16
    assert ok(256, 256, 256, 1, 16, 2, 0) == lib.MXG_ERR_FMT
    assert ok(256, 256, 256, 1, 32, 2, 0) == lib.MXG_ERR_FMT
    assert ok(256, 256, 256, 1, 32, 0, 4) == lib.MXG_ERR_FMT
    assert ok(256, 256, 200, 1, 32, 0, 0) == lib.MXG_ERR_ALIGN       # K % 16
    assert ok(256, 258, 256, 1, 32, 0, 0) == lib.MXG_ERR_ALIGN       # N % 4
    assert ok(1 << 31, 256, 256, 1, 32, 0, 0) == lib.MXG_ERR_SHAPE   # > int32 rows
    assert ok(1 << 30, 1 << 30, 1 << 30, 1 << 20, 32, 0, 0) == lib.MXG_ERR_SHAPE


def test_sf_bytes(lib):
    assert lib.mxgemm_sf_bytes(256, 256, 1, 32) == 2048
    assert lib.mxgemm_sf_bytes(4000, 2048, 1, 16) == 512 * 32 * 32
    assert lib.mxgemm_sf_bytes(7168, 2048, 1, 16) == 917504
    assert lib.mxgemm_sf_bytes(8192, 1536, 1, 32) == 393216
    assert lib.mxgemm_sf_bytes(256, 256, 1, 7) == 0


def test_launch_config_host_only(lib):
    # without a device the choice assumes 256 CUs: 3072 tiles of 256x256 fill them evenly
    tm, tn, g = lib.mxgemm_launch_config(8192, 24576, 1536, 1, 32, with_grid=False)
    assert (tm, tn, g) == (256, 256, None)
    # 64 tiles of 256x256 would leave most CUs idle: 128x128
    tm, tn, _ = lib.mxgemm_launch_config(2048, 2048, 2048, 1, 32, with_grid=False)
    assert (tm, tn) == (128, 128)
    tm, tn, _ = lib.mxgemm_launch_config(4096, 4096, 0, 1, 32, with_grid=False)
    assert (tm, tn) == (128, 128)   # K = 0 stays on the 128x128 kernel


def test_errors_before_device_work(lib):
    c = ctypes.CDLL(lib.LIB_PATH)
    f = c.mxgemm_amax_ex
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    f.argtypes = [vp] * 6 + [i64] * 4 + [ci] * 3 + [ctypes.c_uint, vp]
    f.restype = ci
    good = 0x7F0000000000
    args = [good] * 6
    dims = [256, 256, 256, 1]
    assert f(*([None] + args[1:]), *dims, 32, 0, 0, 0, None) == lib.MXG_ERR_NULL
    assert f(*(args[:5] + [None]), *dims, 32, 0, 0, 0, None) == lib.MXG_ERR_NULL
    assert f(*([good + 8] + args[1:]), *dims, 32, 0, 0, 0, None) == lib.MXG_ERR_ALIGN
    assert f(*(args[:4] + [good + 4] + args[5:]), *dims, 32, 0, 0, 0, None) == lib.MXG_ERR_ALIGN
    assert f(*args, *dims, 32, 0, 0, 1024, None) == lib.MXG_ERR_FLAGS    # unknown bit
    # m-major C: the bf16 datapath, float32 C, M % 4 == 0 (either tile size)
    mm = lib.MXG_FLAG_C_MMAJOR
    assert f(*args, *dims, 32, 0, 0, mm | lib.MXG_FLAG_FP8_MFMA, None) == lib.MXG_ERR_FLAGS
    assert f(*args, *dims, 32, 0, 0, mm | lib.MXG_FLAG_C_BF16, None) == lib.MXG_ERR_FLAGS
    assert f(*args, *dims, 32, 0, 0, mm | lib.MXG_FLAG_C_F16, None) == lib.MXG_ERR_FLAGS
    assert f(*args, *dims, 32, 0, 0, mm | lib.MXG_FLAG_TILE_128, None) == lib.MXG_ERR_DEVICE   # valid; no GPU here
    assert f(*args, 250, 256, 256, 1, 32, 0, 0, mm, None) == lib.MXG_ERR_ALIGN
    # m-major C rows run along M: M is bounded like N (32-bit per-tile store offsets)
    assert f(*args, (1 << 22) - 4, 16, 16, 1, 32, 0, 0, mm, None) != lib.MXG_ERR_SHAPE
    assert f(*args, (1 << 22), 16, 16, 1, 32, 0, 0, mm, None) == lib.MXG_ERR_SHAPE
    assert f(*args, (1 << 22), 16, 16, 1, 32, 0, 0, 0, None) != lib.MXG_ERR_SHAPE    # n-major C: no such bound
    assert f(*args, *dims, 32, 0, 0, 96, None) == lib.MXG_ERR_FLAGS     # both 16-bit C types
    assert f(*args, *dims, 32, 0, 0, 34, None) == lib.MXG_ERR_FLAGS     # 16-bit C with the FP8 datapath
    assert f(*args, *dims, 32, 0, 0, 16, None) == lib.MXG_ERR_FLAGS   # unknown bit
    assert f(*args, *dims, 32, 0, 0, 12, None) == lib.MXG_ERR_FLAGS   # both tile flags
    assert f(*args, 256, 256, 256, 1, 64, 0, 0, 0, None) == lib.MXG_ERR_SFVEC
    assert f(*args, 256, 256, 256, 1, 32, 0, 9, 0, None) == lib.MXG_ERR_FMT
    assert f(*args, 256, 256, 100, 1, 32, 0, 0, 0, None) == lib.MXG_ERR_ALIGN
    assert f(*args, 256, -5, 256, 1, 32, 0, 0, 0, None) == lib.MXG_ERR_SHAPE
    t = c.mxgemm_codes_to_kmajor
    t.argtypes = [vp, vp, i64, i64, i64, vp]
    t.restype = ci
    assert t(good, good, 72, 48, 1, None) == lib.MXG_ERR_ALIGN    # MN % 16
    assert t(good, good, 80, 40, 1, None) == lib.MXG_ERR_ALIGN    # K % 16
    assert t(good + 8, good, 80, 48, 1, None) == lib.MXG_ERR_ALIGN
    assert t(None, good, 80, 48, 1, None) == lib.MXG_ERR_NULL
    assert t(good, good, -16, 48, 1, None) == lib.MXG_ERR_SHAPE
    assert t(None, None, 0, 48, 1, None) == lib.MXG_OK              # nothing to do
    pr = c.mxgemm_proj_rope_mxfp8
    pr.argtypes = [vp] * 7 + [i64] * 4 + [vp]
    pr.restype = ci
    buf7 = [good] * 7
    assert pr(*buf7, 64, 3, 200, 64, None) == lib.MXG_ERR_SHAPE      # head_dim % 32
    assert pr(*buf7, 64, 3, 288, 64, None) == lib.MXG_ERR_SHAPE      # head_dim above 256
    assert pr(*buf7, 64, 3, 192, 63, None) == lib.MXG_ERR_SHAPE      # odd rotary width
    assert pr(*buf7, 64, 3, 192, 160, None) == lib.MXG_ERR_SHAPE     # rotary width above 128
    assert pr(*buf7, 48, 3, 192, 64, None) == lib.MXG_ERR_ALIGN      # tokens % 32
    assert pr(*([good, good + 2] + buf7[2:]), 64, 3, 192, 64, None) == lib.MXG_ERR_ALIGN   # cos
    assert pr(*([None] + buf7[1:]), 64, 3, 192, 64, None) == lib.MXG_ERR_NULL
    assert pr(*([None] * 7), 0, 3, 192, 64, None) == lib.MXG_OK        # nothing to do
    r = c.mxgemm_amax_reset
    r.argtypes = [vp, vp]
    r.restype = ci
    assert r(None, None) == lib.MXG_ERR_NULL


def test_python_errors_map_to_exceptions(lib):
    with pytest.raises(ValueError):
        lib.mxgemm_amax(None, None, None, None, None, None, 16, 16, 16, 1, 32, 0, 0, stream=0)
    assert "sf_vec_size" in lib.mxgemm_strerror(lib.MXG_ERR_SFVEC)
    assert lib.mxgemm_strerror(-99) == "unknown status"


def test_quantize_errors_before_device_work(lib):
    c = ctypes.CDLL(lib.LIB_PATH)
    f = c.mxgemm_mx_quantize
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    f.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
    f.restype = ci
    good = 0x7F0000000000
    assert f(None, good, good, 128, 128, 1, 32, 0, None) == lib.MXG_ERR_NULL
    assert f(good, good, None, 128, 128, 1, 32, 0, None) == lib.MXG_ERR_NULL
    assert f(good + 4, good, good, 128, 128, 1, 32, 0, None) == lib.MXG_ERR_ALIGN
    assert f(good, good, good + 8, 128, 128, 1, 32, 0, None) == lib.MXG_ERR_ALIGN
    assert f(good, good, good, 128, 120, 1, 32, 0, None) == lib.MXG_ERR_ALIGN        # K % 16
    assert f(good, good, good, 128, 128, 1, 64, 0, None) == lib.MXG_ERR_SFVEC
    assert f(good, good, good, 128, 128, 1, 32, 2, None) == lib.MXG_ERR_FMT
    assert f(good, good, good, -1, 128, 1, 32, 0, None) == lib.MXG_ERR_SHAPE
    assert f(good, good, good, 128, 1 << 23, 1, 32, 0, None) == lib.MXG_ERR_SHAPE   # 128 rows past 32-bit offsets
    # empty problems queue nothing and need no pointers
    assert f(None, None, None, 0, 128, 1, 32, 0, None) == lib.MXG_OK
    assert f(None, None, None, 128, 0, 1, 32, 0, None) == lib.MXG_OK
    assert f(None, None, None, 128, 128, 0, 32, 0, None) == lib.MXG_OK


def test_rowwise_repack_errors_before_device_work(lib):
    c = ctypes.CDLL(lib.LIB_PATH)
    f = c.mxgemm_sf_rowwise_to_atoms
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    f.argtypes = [vp, vp, i64, i64, i64, ci, vp]
    f.restype = ci
    good = 0x7F0000000000
    assert f(None, good, 128, 128, 1, 32, None) == lib.MXG_ERR_NULL
    assert f(good, None, 128, 128, 1, 32, None) == lib.MXG_ERR_NULL
    assert f(good, good + 4, 128, 128, 1, 32, None) == lib.MXG_ERR_ALIGN
    assert f(good, good, 128, 128, 1, 8, None) == lib.MXG_ERR_SFVEC
    assert f(good, good, -3, 128, 1, 32, None) == lib.MXG_ERR_SHAPE
    assert f(None, None, 0, 128, 1, 32, None) == lib.MXG_OK


def test_plan_validation_before_device_work(lib):
    c = ctypes.CDLL(lib.LIB_PATH)
    init, ex = c.mxgemm_plan_init, c.mxgemm_plan_execute
    vp, i64, ci, cu = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint
    init.argtypes = [vp, i64, i64, i64, i64, ci, ci, ci, cu]
    init.restype = ci
    ex.argtypes = [vp] * 8
    ex.restype = ci
    plan = (ctypes.c_uint64 * 32)()
    assert init(None, 256, 256, 256, 1, 32, 0, 0, 0) == lib.MXG_ERR_NULL
    assert init(plan, 256, 256, 200, 1, 32, 0, 0, 0) == lib.MXG_ERR_ALIGN
    assert init(plan, 256, 256, 256, 1, 64, 0, 0, 0) == lib.MXG_ERR_SFVEC
    assert init(plan, 256, 256, 256, 1, 32, 0, 0, 96) == lib.MXG_ERR_FLAGS
    # packed FP4 at sf = 16 runs 128x128 tiles only
    assert init(plan, 256, 256, 256, 1, 16, 2, 2, lib.MXG_FLAG_TILE_256) == lib.MXG_ERR_FLAGS
    # m-major A / n-major B: 8-bit codes, bf16 datapath, float32 n-major C, whole 16-byte chunks
    am, bn = lib.MXG_FLAG_A_MMAJOR, lib.MXG_FLAG_B_NMAJOR
    assert init(plan, 256, 256, 256, 1, 32, 2, 2, am) == lib.MXG_ERR_FLAGS
    assert init(plan, 256, 256, 256, 1, 32, 0, 0, bn | lib.MXG_FLAG_FP8_MFMA) == lib.MXG_ERR_FLAGS
    assert init(plan, 256, 256, 256, 1, 32, 0, 0, am | lib.MXG_FLAG_C_BF16) == lib.MXG_ERR_FLAGS
    assert init(plan, 256, 256, 256, 1, 32, 0, 0, am | lib.MXG_FLAG_C_MMAJOR) == lib.MXG_ERR_FLAGS
    assert init(plan, 264, 256, 256, 1, 32, 0, 0, am) == lib.MXG_ERR_ALIGN
    assert init(plan, 256, 264, 256, 1, 32, 0, 0, bn) == lib.MXG_ERR_ALIGN
    assert init(plan, 264, 256, 256, 1, 32, 0, 0, bn) != lib.MXG_ERR_ALIGN     # M is free with B n-major
    assert init(plan, 1 << 16, 256, 1 << 15, 1, 32, 0, 0, am) == lib.MXG_ERR_SHAPE  # one batch >= 2^31 B
    assert init(plan, 1 << 16, 256, 1 << 15, 1, 32, 0, 0, bn) != lib.MXG_ERR_SHAPE
    assert init(plan, -1, 256, 256, 1, 32, 0, 0, 0) == lib.MXG_ERR_SHAPE
    assert init(plan, 1 << 22, 16, 16, 1, 32, 0, 0, lib.MXG_FLAG_C_MMAJOR) == lib.MXG_ERR_SHAPE
    # a plan that was never initialised is refused before any device call
    zero = (ctypes.c_uint64 * 32)()
    good = 0x7F0000000000
    assert ex(zero, good, good, good, good, good, good, None) == lib.MXG_ERR_NULL
    assert ex(None, good, good, good, good, good, good, None) == lib.MXG_ERR_NULL


def test_projection_errors_before_device_work(lib):
    c = ctypes.CDLL(lib.LIB_PATH)
    vp, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    wsb = c.mxgemm_projection_workspace_bytes
    wsb.argtypes = [i64] * 4
    wsb.restype = sz
    ws_call = c.mxgemm_projection_mxfp8
    ws_call.argtypes = [vp] * 10 + [i64] * 5 + [vp, sz, vp]
    ws_call.restype = ci
    na = c.mxgemm_projection_mxfp8_noalloc
    na.argtypes = [vp] * 10 + [i64] * 5 + [vp]
    na.restype = ci
    good = 0x7F0000000000
    ptrs = [good] * 10
    # workspace = x's atoms (rounded up to 256 bytes) + w's atoms, 512 bytes per 128 rows x 128 K
    assert wsb(4096, 128, 192, 1536) == 512 * 32 * 12 + 512 * 192 * 12
    assert wsb(96, 4, 192, 160) == 512 * 1 * 2 + 512 * 6 * 2
    assert wsb(-1, 4, 192, 160) == 0
    # the fixed scratch of the allocation-free entry: the largest problem that fits is accepted by the
    # size check (and reaches the pointer checks), one that does not is refused before any device call
    cap = lib.MXGEMM_NOALLOC_SCRATCH_BYTES
    assert wsb(4096, 128, 192, 7168) <= cap
    assert na(*([None] * 10), 4096, 128, 192, 64, 7168, None) == lib.MXG_ERR_NULL
    assert wsb(16384, 128, 192, 7168) > cap
    assert na(*ptrs, 16384, 128, 192, 64, 7168, None) == lib.MXG_ERR_SCRATCH
    assert na(*([None] * 10), 16384, 128, 192, 64, 7168, None) == lib.MXG_ERR_SCRATCH
    # shape rules shared by both entries come first
    for bad in ((96, 4, 100, 64, 160), (96, 4, 192, 72, 160), (100, 4, 192, 64, 160), (96, 4, 192, 64, 0)):
        st = na(*ptrs, *bad, None)
        assert st in (lib.MXG_ERR_SHAPE, lib.MXG_ERR_ALIGN), bad
        assert ws_call(*ptrs, *bad, good, 1 << 20, None) == st, bad
    # empty problems need no pointers
    assert na(*([None] * 10), 0, 4, 192, 64, 160, None) == lib.MXG_OK
    assert ws_call(*([None] * 10), 0, 4, 192, 64, 160, None, 0, None) == lib.MXG_OK
    # a short or misaligned caller workspace
    need = wsb(96, 4, 192, 160)
    assert ws_call(*ptrs, 96, 4, 192, 64, 160, good, need - 1, None) == lib.MXG_ERR_SHAPE
    assert ws_call(*ptrs, 96, 4, 192, 64, 160, good + 16, need, None) == lib.MXG_ERR_ALIGN
    assert ws_call(*ptrs, 96, 4, 192, 64, 160, None, need, None) == lib.MXG_ERR_NULL
