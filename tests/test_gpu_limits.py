"""GPU parity at the largest shapes the products accept: rows of 2^26
elements for the matvec (n <= 8, and its passes, which 9..128 columns may
take; its 32-bit buffer offsets reach 2^31 bytes per super-tile stream) and
of 2^22 elements for the wide contraction, in both formats; one block past
either limit is rejected on the host (tests/test_abi_host.py).  The wide
case runs 129 columns, which only the wide product takes: the product
shape's two column tiles, the second at an offset of 2^30 bytes into X;
the narrower shapes' offsets are bounded by the product shape's."""
import numpy as np
import pytest
import torch

import oracle
import block_scaled_bit_nvfp4_amd as nv
from tests import _gpu as G

pytestmark = pytest.mark.gpu

MAX_NARROW_COLS = 1 << 26
MAX_WIDE_COLS = 1 << 22


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load()
    yield
    torch.cuda.synchronize()


def _run(fmt, R, K, n, seed):
    W = G.seeded_matrix(R, K, seed)
    X = G.seeded_x(n, K, seed=seed + 1)
    Y = torch.full((n, R), float("nan"), dtype=torch.float32, device=G.DEV)
    codes = torch.empty(R, K // 2, dtype=torch.uint8, device=G.DEV)
    if fmt == "mxfp4":
        scales = torch.empty(R, K // 32, dtype=torch.uint8, device=G.DEV)
        nv.mxfp4_quantize(W, R, K, 1.0, codes, scales)
        wq, ws = nv.alloc_mx_repacked(R, K, G.DEV)
        nv.mxfp4_repack(codes, scales, R, K, wq, ws)
        nv.mxfp4_gemv(wq, ws, 1.0, R, K, X, n, Y)
        c_ref, s_ref = oracle.mx_quantize(W.cpu().numpy(), 1.0)
        Y_ref, S = oracle.mx_gemv(c_ref, s_ref, 1.0, G.wl.bf16_bits(X))
    else:
        scales = torch.empty(R, K // 16, dtype=torch.uint8, device=G.DEV)
        nv.nvfp4_quantize(W, R, K, 1.0, codes, scales)
        wq, ws = nv.alloc_repacked(R, K, G.DEV)
        nv.nvfp4_repack(codes, scales, R, K, wq, ws)
        nv.nvfp4_gemv(wq, ws, 1.0, R, K, X, n, Y)
        c_ref, s_ref = oracle.quantize(W.cpu().numpy(), 1.0)
        Y_ref, S = oracle.gemv(c_ref, s_ref, 1.0, G.wl.bf16_bits(X))
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    G.assert_within_tolerance(Y.cpu().numpy(), Y_ref, S, "%s %dx%d n=%d" % (fmt, R, K, n))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("n", [1, 3])
def test_narrow_at_max_cols(fmt, n):
    G.note("limits narrow %s 1x%d n=%d" % (fmt, MAX_NARROW_COLS, n))
    _run(fmt, 1, MAX_NARROW_COLS, n, 101 + n)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_matvec_passes_at_max_cols(fmt):
    """Ten columns: two passes of the matvec, the second reading X and
    writing Y 8 rows in (an offset of 2^30 bytes into X)."""
    G.note("limits passes %s 1x%d n=10" % (fmt, MAX_NARROW_COLS))
    _run(fmt, 1, MAX_NARROW_COLS, 10, 111)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_wide_at_max_cols(fmt):
    G.note("limits wide %s 16x%d n=129" % (fmt, MAX_WIDE_COLS))
    _run(fmt, 16, MAX_WIDE_COLS, 129, 201)
