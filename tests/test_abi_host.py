"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/nvfp4.h declares, computes plane sizes, and rejects
bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import block_scaled_bit_nvfp4_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

OK, EINVAL, ESHAPE, EALIGN, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nv.library_path()):
        from block_scaled_bit_nvfp4_amd import build
        build.build(verbose=False)
    return nv.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("nvfp4_repack", "nvfp4_gemv", "nvfp4_gemv_argmax", "nvfp4_quantize",
                 "nvfp4_dequant", "nvfp4_swiglu", "nvfp4_strerror"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    # and nothing from the internal namespace leaks as a C symbol
    for internal in ("launch_narrow", "narrow_config", "launch_mfma"):
        with pytest.raises(AttributeError):
            getattr(lib, internal)


def test_binding_names_match_header():
    for name in declared_functions():
        assert callable(getattr(nv, name)), name


@pytest.mark.parametrize("rows,cols,code,scale", [
    # (64-row super-tiles) x (octets of 8 blocks) x (4096 | 512) bytes
    (256, 512, 4 * 4 * 4096, 4 * 4 * 512),
    (4096, 4096, 64 * 32 * 4096, 64 * 32 * 512),
    (17, 32, 1 * 1 * 4096, 1 * 1 * 512),
    (151936, 5120, 2374 * 40 * 4096, 2374 * 40 * 512),
    (5120, 17408, 80 * 136 * 4096, 80 * 136 * 512),
    (65, 144, 2 * 2 * 4096, 2 * 2 * 512),
])
def test_plane_sizes(lib, rows, cols, code, scale):
    assert nv.nvfp4_repacked_code_bytes(rows, cols) == code
    assert nv.nvfp4_repacked_scale_bytes(rows, cols) == scale


@pytest.mark.parametrize("rows,cols", [(0, 512), (16, 0), (16, 8), (16, 24), (-1, 16), (16, 1 << 40)])
def test_plane_sizes_invalid(lib, rows, cols):
    assert nv.nvfp4_repacked_code_bytes(rows, cols) == 0
    assert nv.nvfp4_repacked_scale_bytes(rows, cols) == 0


def test_workspace_bytes(lib):
    # a 1152-byte header for the finish (a 128-byte counter line, then 16
    # workgroups x 8 columns of partial maxima), then one 64-bit key per
    # workgroup and column: a 16 x 32 matrix runs 4 one-tile workgroups (its
    # 64-row super-tile), the 151936 x 5120 vocabulary projection (9496 tiles)
    # 4748 two-tile workgroups at one to three columns and, from four columns
    # (the argmax's own rule at four), 2374 four-tile ones; the 17408 x 5120
    # matrix (1088 tiles) 1088 one-tile workgroups
    H = 1152
    assert [nv.nvfp4_gemv_argmax_workspace_bytes(16, 32, n) for n in (0, 1, 4, 8, 9)] == [0, H + 32, H + 128,
                                                                                           H + 256, 0]
    assert nv.nvfp4_gemv_argmax_workspace_bytes(151936, 5120, 1) == H + 4748 * 1 * 8
    assert nv.nvfp4_gemv_argmax_workspace_bytes(151936, 5120, 3) == H + 4748 * 3 * 8
    assert nv.nvfp4_gemv_argmax_workspace_bytes(151936, 5120, 4) == H + 2374 * 4 * 8
    assert nv.nvfp4_gemv_argmax_workspace_bytes(17408, 5120, 4) == H + 1088 * 4 * 8     # 1088 tiles: one each
    assert nv.nvfp4_gemv_argmax_workspace_bytes(17408, 5120, 1) == H + 1088 * 8
    # 257..512 tiles: one tile per workgroup while a row has at most 32
    # octets (the 8192 x 4096 draft head), two tiles otherwise
    assert nv.nvfp4_gemv_argmax_workspace_bytes(8192, 4096, 1) == H + 512 * 8
    assert nv.nvfp4_gemv_argmax_workspace_bytes(8192, 5120, 1) == H + 256 * 8
    assert nv.nvfp4_gemv_argmax_workspace_bytes(5120, 17408, 1) == H + 160 * 8
    # the two-tile parity shapes: 261 tiles with 33-octet rows, and 4100 tiles
    assert nv.nvfp4_gemv_argmax_workspace_bytes(4176, 4112, 1) == H + 66 * 2 * 8
    assert nv.nvfp4_gemv_argmax_workspace_bytes(65600, 528, 1) == H + 1025 * 2 * 8
    # past four columns the tiles per workgroup double, except for small
    # matrices and the two-tile shapes of 257..512 tiles
    assert nv.nvfp4_gemv_argmax_workspace_bytes(151936, 5120, 5) == H + 2374 * 5 * 8
    assert nv.nvfp4_gemv_argmax_workspace_bytes(17408, 5120, 8) == H + 544 * 8 * 8
    assert nv.nvfp4_gemv_argmax_workspace_bytes(8192, 4096, 6) == H + 256 * 6 * 8
    assert nv.nvfp4_gemv_argmax_workspace_bytes(4096, 4096, 8) == H + 256 * 8 * 8
    assert nv.nvfp4_gemv_argmax_workspace_bytes(5120, 17408, 8) == H + 160 * 8 * 8
    assert nv.nvfp4_gemv_argmax_workspace_bytes(16, 24, 4) == 0
    # the bound the header states: the header plus 4 bytes per row, rows
    # rounded up to 64
    for R, K in ((1, 16), (16, 32), (65, 512), (4176, 2064), (65620, 528), (151936, 5120)):
        for n in range(1, 9):
            assert 0 < nv.nvfp4_gemv_argmax_workspace_bytes(R, K, n) <= H + 4 * (-(-R // 64) * 64), (R, K, n)
    assert nv.nvfp4_gemv_argmax_workspace_bytes(16, (1 << 26) + 16, 4) == 0


def test_noalloc_array_covers_every_shape_up_to_262144_rows(lib):
    """The static array of the allocation-free argmax (1 MiB) holds the
    workspace of every n <= 8 up to 262144 rows: each rows class of the
    decomposition (small, short-row, 257..512, 513..4096 and more tiles) at
    its edges and at the limit, for short and long rows."""
    worst = 0
    rows = sorted({r for t in (1, 256, 257, 512, 513, 4096, 4097, 16384) for r in (16 * t - 15, 16 * t)} |
                  {262144 - 63, 262144})
    for R in rows:
        for K in (16, 512, 528, 4096, 5120, 17408):
            for n in range(1, 9):
                worst = max(worst, nv.nvfp4_gemv_argmax_workspace_bytes(R, K, n))
    assert 0 < worst <= 1 << 20
    # the largest row count at n = 8: 16366 four-tile workgroups of 64 rows
    # fill the array with the header exactly
    assert nv.nvfp4_gemv_argmax_workspace_bytes(1047424, 16, 8) == 1 << 20


@pytest.mark.parametrize("rows,cols,code,scale", [
    (256, 512, 4 * 4 * 4096, 4 * 4 * 256),
    (17, 32, 1 * 1 * 4096, 1 * 1 * 256),
    (17408, 5120, 272 * 40 * 4096, 272 * 40 * 256),
    (65, 160, 2 * 2 * 4096, 2 * 2 * 256),
])
def test_mx_plane_sizes(lib, rows, cols, code, scale):
    assert nv.mxfp4_repacked_code_bytes(rows, cols) == code == nv.nvfp4_repacked_code_bytes(rows, cols)
    assert nv.mxfp4_repacked_scale_bytes(rows, cols) == scale


@pytest.mark.parametrize("rows,cols", [(16, 16), (16, 48), (0, 32), (16, 0)])
def test_mx_plane_sizes_invalid(lib, rows, cols):
    assert nv.mxfp4_repacked_code_bytes(rows, cols) == 0
    assert nv.mxfp4_repacked_scale_bytes(rows, cols) == 0


def test_mx_validation(lib):
    assert lib.mxfp4_gemv(A, B, 1.0, 16, 48, C, 1, A, S0) == ESHAPE       # cols % 32
    assert lib.mxfp4_gemv(A, B, 1.0, 16, 64, C, 0, A, S0) == EINVAL
    assert lib.mxfp4_gemv(MIS, B, 1.0, 16, 64, C, 1, A, S0) == EALIGN
    assert lib.mxfp4_quantize(A, 16, 48, 1.0, B, C, S0) == ESHAPE
    assert lib.mxfp4_quantize(A, 16, 64, 0.0, B, C, S0) == EINVAL
    assert lib.mxfp4_repack(A, B, 16, 48, C, A, S0) == ESHAPE
    assert lib.mxfp4_repack(A, B, 16, 64, C, MIS, S0) == EALIGN
    assert lib.mxfp4_dequant(A, B, 1.0, 16, 64, NULL, NULL, S0) == EINVAL


def test_strerror(lib):
    for code in (OK, EINVAL, ESHAPE, EALIGN, EWORKSPACE, EHIP):
        assert nv.nvfp4_strerror(code)
    assert nv.nvfp4_strerror(OK) == "ok"
    assert nv.nvfp4_strerror(12345) == "unknown status"


# Fake device addresses: validation rejects these calls before any HIP call,
# so nothing is ever dereferenced or launched.
A = ctypes.c_void_p(0x100000)       # 16-byte aligned
B = ctypes.c_void_p(0x200000)
C = ctypes.c_void_p(0x300000)
MIS = ctypes.c_void_p(0x100008)     # 8-byte aligned only
NULL = None
S0 = None


def test_gemv_validation(lib):
    g = lib.nvfp4_gemv
    assert g(NULL, B, 1.0, 16, 32, C, 1, A, S0) == EINVAL
    assert g(A, B, 1.0, 16, 32, C, 0, A, S0) == EINVAL          # n = 0
    assert g(A, B, 1.0, 16, 32, C, 65537, A, S0) == EINVAL      # n too large
    assert g(A, B, 0.0, 16, 32, C, 1, A, S0) == EINVAL          # tscale <= 0
    assert g(A, B, float("nan"), 16, 32, C, 1, A, S0) == EINVAL
    assert g(A, B, float("inf"), 16, 32, C, 1, A, S0) == EINVAL
    assert g(A, B, 1.0, 0, 32, C, 1, A, S0) == ESHAPE
    assert g(A, B, 1.0, 16, 40, C, 1, A, S0) == ESHAPE
    assert g(MIS, B, 1.0, 16, 32, C, 1, A, S0) == EALIGN
    assert g(A, B, 1.0, 16, 32, MIS, 1, A, S0) == EALIGN
    assert g(A, B, 1.0, 16, 32, C, 1, ctypes.c_void_p(0x100002), S0) == EALIGN
    assert g(A, B, 1.0, 16, 32, C, 1, NULL, S0) == EINVAL
    # the matvec (n <= 8, and its passes, which 9..128 columns may take) takes
    # rows of at most 2^26 elements, the wide product rows of at most 2^22;
    # past 128 columns only the wide product runs.  Every call here must fail
    # validation: nothing may launch.  (9..128 columns with rows between 2^22
    # and 2^26 elements are valid: they run as passes.)
    assert g(A, B, 1.0, 16, (1 << 26) + 16, C, 8, A, S0) == ESHAPE
    assert g(A, B, 1.0, 16, (1 << 26) + 16, C, 16, A, S0) == ESHAPE    # passes impossible, wide too wide
    assert g(A, B, 1.0, 16, (1 << 26) + 16, C, 128, A, S0) == ESHAPE
    assert g(A, B, 1.0, 16, (1 << 22) + 32, C, 129, A, S0) == ESHAPE   # wide only, too wide
    assert lib.mxfp4_gemv(A, B, 1.0, 16, (1 << 26) + 32, C, 8, A, S0) == ESHAPE
    assert lib.mxfp4_gemv(A, B, 1.0, 16, (1 << 26) + 32, C, 16, A, S0) == ESHAPE
    assert lib.mxfp4_gemv(A, B, 1.0, 16, (1 << 22) + 32, C, 129, A, S0) == ESHAPE


def test_argmax_validation(lib):
    g = lib.nvfp4_gemv_argmax
    assert g(A, B, 1.0, 16, 32, C, 4, NULL, A, B, 127, S0) == EWORKSPACE
    assert g(A, B, 1.0, 16, 32, C, 9, NULL, A, B, 1024, S0) == EINVAL   # argmax is n <= 8
    assert g(A, B, 1.0, 16, 32, C, 4, NULL, NULL, B, 128, S0) == EINVAL
    assert g(A, B, 1.0, 16, 32, C, 4, NULL, A, NULL, 128, S0) == EINVAL
    assert g(A, B, 1.0, 16, 32, C, 4, NULL, A, ctypes.c_void_p(0x200004), 128, S0) == EALIGN


def test_other_entry_points_validation(lib):
    assert lib.nvfp4_quantize(A, 16, 32, 1.0, B, NULL, S0) == EINVAL
    assert lib.nvfp4_quantize(A, 16, 33, 1.0, B, C, S0) == ESHAPE
    assert lib.nvfp4_quantize(A, 16, 32, -1.0, B, C, S0) == EINVAL
    assert lib.nvfp4_quantize(MIS, 16, 32, 1.0, B, C, S0) == EALIGN
    assert lib.nvfp4_repack(A, B, 16, 32, C, NULL, S0) == EINVAL
    assert lib.nvfp4_repack(A, B, 16, 32, C, MIS, S0) == EALIGN
    assert lib.nvfp4_repack(A, B, 16, 0, C, A, S0) == ESHAPE
    assert lib.nvfp4_dequant(A, B, 1.0, 16, 32, NULL, NULL, S0) == EINVAL
    assert lib.nvfp4_dequant(A, B, 1.0, 16, 32, MIS, NULL, S0) == EALIGN
    assert lib.nvfp4_swiglu(A, 0, 1, B, S0) == ESHAPE
    assert lib.nvfp4_swiglu(A, 16, 0, B, S0) == EINVAL
    assert lib.nvfp4_swiglu(MIS, 16, 1, B, S0) == EALIGN


def test_one_dimensional_grids_past_the_largest_are_rejected(lib):
    """Shapes the layout admits but whose one-workgroup-per-256-items launch
    would pass 2^31 - 1 workgroups get NVFP4_ESHAPE instead of a truncated
    grid (every call here is far past the limit, so nothing launches)."""
    R, K = (1 << 31) - 64, (1 << 31) - 1024          # the largest admitted rows and columns
    assert lib.nvfp4_repacked_code_bytes(R, K) > 0    # a valid layout...
    for f in (lib.nvfp4_quantize, lib.mxfp4_quantize):
        assert f(A, R, K, 1.0, B, C, S0) == ESHAPE
    # just past the limit: 2^39 + 2^20 blocks of 16 (NVFP4), 2^39 + 2^21 of 32 (MXFP4)
    assert lib.nvfp4_quantize(A, 1 << 20, (1 << 23) + 32, 1.0, B, C, S0) == ESHAPE
    assert lib.mxfp4_quantize(A, 1 << 21, (1 << 23) + 32, 1.0, B, C, S0) == ESHAPE
    for f in (lib.nvfp4_repack, lib.mxfp4_repack):
        assert f(A, B, R, K, C, A, S0) == ESHAPE
    for f in (lib.nvfp4_dequant, lib.mxfp4_dequant):
        assert f(A, B, 1.0, R, K, C, NULL, S0) == ESHAPE
    assert lib.nvfp4_swiglu(A, 1 << 40, 65536, B, S0) == ESHAPE


def test_gemv_swiglu_validation(lib):
    f = lib.nvfp4_gemv_swiglu
    assert f(A, B, 1.0, 512, 1024, C, 1, NULL, NULL, S0) == EINVAL      # h
    assert f(A, B, 1.0, 512, 1000, C, 1, NULL, A, S0) == ESHAPE         # F % 16
    assert f(A, B, 1.0, 40, 1024, C, 1, NULL, A, S0) == ESHAPE          # hidden % 16
    assert f(A, B, 1.0, 512, 1024, C, 9, NULL, A, S0) == EINVAL         # n > 8
    assert f(A, B, 0.0, 512, 1024, C, 1, NULL, A, S0) == EINVAL
    assert f(MIS, B, 1.0, 512, 1024, C, 1, NULL, A, S0) == EALIGN
    assert f(A, B, 1.0, 512, 1024, C, 1, ctypes.c_void_p(0x100002), A, S0) == EALIGN


# ------------------------------------------------ Python binding validation
# The binding checks every tensor before its pointer reaches the library:
# type, contiguity, dtype, the bytes the call's shape implies, and that all
# of them sit on one GPU.  On this host no tensor is on a GPU, so each case
# below is rejected by the first check it fails, which the message names.

import torch  # noqa: E402


def _t(nbytes, dtype=torch.uint8):
    return torch.zeros(max(1, nbytes // torch.tensor([], dtype=dtype).element_size()), dtype=dtype)


def test_binding_rejects_wrong_dtype(lib):
    R, K = 64, 512
    wq, ws = _t(nv.nvfp4_repacked_code_bytes(R, K)), _t(nv.nvfp4_repacked_scale_bytes(R, K))
    X32 = torch.zeros(1, K, dtype=torch.float32)                  # fp32 activations
    Y = torch.zeros(1, R, dtype=torch.float32)
    with pytest.raises(ValueError, match="X: dtype"):
        nv.nvfp4_gemv(wq, ws, 1.0, R, K, X32, 1, Y)
    X = torch.zeros(1, K, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="Y: dtype"):
        nv.nvfp4_gemv(wq, ws, 1.0, R, K, X, 1, Y.to(torch.float64))
    with pytest.raises(ValueError, match="wq: dtype"):
        nv.nvfp4_gemv(wq.to(torch.int32), ws, 1.0, R, K, X, 1, Y)
    with pytest.raises(ValueError, match="argmax: dtype"):
        nv.nvfp4_gemv_argmax(wq, ws, 1.0, R, K, X, 1, None, torch.zeros(1, dtype=torch.int64), _t(64))


def test_binding_rejects_short_buffers(lib):
    R, K = 64, 512
    wq, ws = _t(nv.nvfp4_repacked_code_bytes(R, K)), _t(nv.nvfp4_repacked_scale_bytes(R, K))
    X = torch.zeros(4, K, dtype=torch.bfloat16)
    Y = torch.zeros(4, R, dtype=torch.float32)
    with pytest.raises(ValueError, match="X holds"):
        nv.nvfp4_gemv(wq, ws, 1.0, R, K, X[:2].contiguous(), 4, Y)   # n = 4 columns claimed, 2 given
    with pytest.raises(ValueError, match="Y holds"):
        nv.nvfp4_gemv(wq, ws, 1.0, R, K, X, 4, Y[:3].contiguous())
    with pytest.raises(ValueError, match="wq holds"):
        nv.nvfp4_gemv(wq[:-1].contiguous(), ws, 1.0, R, K, X, 4, Y)
    with pytest.raises(ValueError, match="ws holds"):
        nv.mxfp4_gemv(wq, _t(nv.mxfp4_repacked_scale_bytes(R, K) - 16), 1.0, R, K, X, 4, Y)
    with pytest.raises(ValueError, match="h holds"):
        nv.nvfp4_swiglu(torch.zeros(1, 64, dtype=torch.float32), 32, 1, torch.zeros(31, dtype=torch.int16))
    with pytest.raises(ValueError, match="scales holds"):
        nv.nvfp4_quantize(torch.zeros(R, K), R, K, 1.0, _t(R * K // 2), _t(R * K // 16 - 1))


def test_binding_rejects_host_and_strided_tensors(lib):
    R, K = 64, 512
    wq, ws = _t(nv.nvfp4_repacked_code_bytes(R, K)), _t(nv.nvfp4_repacked_scale_bytes(R, K))
    X = torch.zeros(1, K, dtype=torch.bfloat16)
    Y = torch.zeros(1, R, dtype=torch.float32)
    with pytest.raises(ValueError, match="must be in GPU memory"):
        nv.nvfp4_gemv(wq, ws, 1.0, R, K, X, 1, Y)
    with pytest.raises(ValueError, match="contiguous"):
        nv.nvfp4_gemv(wq, ws, 1.0, R, K, torch.zeros(K, 2, dtype=torch.bfloat16).t(), 1, Y)
    with pytest.raises(TypeError):
        nv.nvfp4_gemv(wq, ws, 1.0, R, K, [0] * K, 1, Y)
    with pytest.raises(ValueError, match="is required"):
        nv.nvfp4_gemv(wq, ws, 1.0, R, K, X, 1, None)


def test_argmax_noalloc_validation(lib):
    g = lib.nvfp4_gemv_argmax_noalloc
    # the header and the keys of 1047424 rows at n = 8 fill the 1 MiB array;
    # one row more is rejected before any HIP call
    assert g(A, B, 1.0, 1047424 + 1, 16, C, 8, NULL, A, S0) == EWORKSPACE
    assert g(A, B, 1.0, 16, 32, C, 9, NULL, A, S0) == EINVAL      # argmax is n <= 8
    assert g(A, B, 1.0, 16, 32, C, 4, NULL, NULL, S0) == EINVAL
    assert g(A, B, 1.0, 16, 32, C, 4, ctypes.c_void_p(0x300002), A, S0) == EALIGN
    assert g(MIS, B, 1.0, 16, 32, C, 4, NULL, A, S0) == EALIGN


class _Prod(ctypes.Structure):
    _fields_ = [("wq", ctypes.c_void_p), ("ws", ctypes.c_void_p), ("tscale", ctypes.c_float),
                ("rows", ctypes.c_int64), ("y", ctypes.c_void_p), ("argmax", ctypes.c_void_p)]


def _prods(*items):
    arr = (_Prod * len(items))()
    for i, (rows, y, am) in enumerate(items):
        arr[i] = _Prod(A, B, 1.0, rows, y, am)
    return arr


def test_batch_workspace_and_validation(lib):
    lib.nvfp4_gemv_batch_workspace_bytes.restype = ctypes.c_size_t
    lib.nvfp4_gemv_batch_workspace_bytes.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int]
    lib.nvfp4_gemv_batch.restype = ctypes.c_int
    lib.nvfp4_gemv_batch.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    wsb = lib.nvfp4_gemv_batch_workspace_bytes
    # the verify pair at n = 4 runs as one launch with the argmax head's four
    # tiles per workgroup: its 2374 super-tiles give 2374 workgroups x 4 keys,
    # after the head's 1152-byte finish header
    pair = _prods((151936, C, A), (17408, C, NULL))
    assert wsb(pair, 2, 5120, 4) == 1152 + 2374 * 4 * 8
    # no argmax: no workspace
    assert wsb(_prods((4096, C, NULL)), 1, 4096, 1) == 0
    # one launch at the larger product's two tiles per workgroup: the
    # 9000-row product's 141 super-tiles give 282 workgroups, not its own 564
    assert wsb(_prods((70000, C, A), (9000, C, A)), 2, 2048, 1) == 2 * 1152 + (2188 + 282) * 8
    # 8 against 16 waves a row: each product's own decomposition
    mixed = _prods((9000, C, A), (700, C, A))
    assert wsb(mixed, 2, 2048, 3) == (nv.nvfp4_gemv_argmax_workspace_bytes(9000, 2048, 3) +
                                      nv.nvfp4_gemv_argmax_workspace_bytes(700, 2048, 3))
    g = lib.nvfp4_gemv_batch
    assert g(pair, 0, 5120, C, 4, B, 1 << 20, S0) == EINVAL            # count
    assert g(pair, 5, 5120, C, 4, B, 1 << 20, S0) == EINVAL
    assert g(pair, 2, 5120, C, 9, B, 1 << 20, S0) == EINVAL            # n > 8
    assert g(pair, 2, 5120, NULL, 4, B, 1 << 20, S0) == EINVAL         # X
    assert g(pair, 2, 5120, MIS, 4, B, 1 << 20, S0) == EALIGN
    assert g(pair, 2, 5128, C, 4, B, 1 << 20, S0) == ESHAPE            # cols % 16
    assert g(pair, 2, 5120, C, 4, B, 1152 + 2374 * 4 * 8 - 1, S0) == EWORKSPACE
    assert g(pair, 2, 5120, C, 4, NULL, 1 << 20, S0) == EINVAL         # workspace needed
    assert g(_prods((64, NULL, NULL)), 1, 512, C, 1, NULL, 0, S0) == EINVAL   # neither y nor argmax
    assert g(_prods((64, ctypes.c_void_p(0x300002), NULL)), 1, 512, C, 1, NULL, 0, S0) == EALIGN
    assert g(_prods((0, C, NULL)), 1, 512, C, 1, NULL, 0, S0) == ESHAPE


def test_binding_batch_checks_every_product(lib):
    R, K, n = 64, 512, 2
    wq, ws = _t(nv.nvfp4_repacked_code_bytes(R, K)), _t(nv.nvfp4_repacked_scale_bytes(R, K))
    X = torch.zeros(n, K, dtype=torch.bfloat16)
    ok = dict(wq=wq, ws=ws, tscale=1.0, rows=R, y=torch.zeros(n, R), argmax=None)
    with pytest.raises(ValueError, match=r"products\[1\].ws holds"):
        nv.nvfp4_gemv_batch([ok, dict(ok, ws=ws[:-1].contiguous())], K, X, n)
    with pytest.raises(ValueError, match=r"products\[0\].argmax: dtype"):
        nv.nvfp4_gemv_batch([dict(ok, argmax=torch.zeros(n, dtype=torch.int64))], K, X, n)
    with pytest.raises(ValueError, match=r"products\[0\].y holds"):
        nv.nvfp4_gemv_batch([dict(ok, y=torch.zeros(n, R - 1))], K, X, n)
    with pytest.raises(ValueError, match="must be in GPU memory"):
        nv.nvfp4_gemv_batch([ok], K, X, n)


PROBE_HEADER = os.path.join(ROOT, "include", "nvfp4_probe.h")


def test_probe_library_exports_its_header_and_checks_arguments():
    """libnvfp4_probe (the measured walls) exports every function
    include/nvfp4_probe.h declares; the read-and-store probe rejects bad
    arguments on the host (no call here passes validation, so none launches)."""
    path = os.path.join(ROOT, "block_scaled_bit_nvfp4_amd", "libnvfp4_probe.so")
    if not os.path.exists(path):
        from block_scaled_bit_nvfp4_amd import build
        build.build(verbose=False)
    plib = ctypes.CDLL(path)
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(nvfp4_probe_\w+)\s*\(", text)))
    assert "nvfp4_probe_stream_read_store" in names
    for name in names:
        assert hasattr(plib, name), name
    f = plib.nvfp4_probe_stream_read_store
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    buf, out, mis = ctypes.c_void_p(0x200000), ctypes.c_void_p(0x400000), ctypes.c_void_p(0x200004)
    assert f(None, 4096, out, 4096, 8, None) == EINVAL
    assert f(buf, 4096, None, 4096, 8, None) == EINVAL
    assert f(buf, 4096, out, 4096, 0, None) == EINVAL             # groups
    assert f(buf, 4096, out, 4096, 65537, None) == EINVAL
    assert f(buf, 8, out, 4096, 8, None) == ESHAPE                # read size
    assert f(buf, 1 << 31, out, 4096, 8, None) == ESHAPE
    assert f(buf, 4096, out, 4100, 8, None) == ESHAPE             # output not a multiple of 16
    assert f(buf, 4096, out, 0, 8, None) == ESHAPE
    assert f(mis, 4096, out, 4096, 8, None) == EALIGN
    assert f(buf, 4096, mis, 4096, 8, None) == EALIGN
