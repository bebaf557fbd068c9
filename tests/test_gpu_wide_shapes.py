"""The wide product's narrower workgroup shapes (one tile per wave, two
super-tiles, 32, 64 or 128 columns), which serve 9 to 128 columns on
matrices large enough that the wide product beats passes of the matvec.

Each output is the same MFMA chain over the same k order in every shape, so
the columns of a product at any width equal, bit for bit, the same columns
of a wider product; the widest here runs the product shape and is checked
against the oracle on sampled rows.  Each shape also repeats its bits over
forty launches (a direct-to-LDS load still in flight at a barrier would
show as an occasional differing launch).  On a matrix too small for the
wide product to pay, 9..128 columns run as passes of the matvec, whose
columns each equal their one-column product."""
import numpy as np
import pytest
import torch

import oracle
import block_scaled_bit_nvfp4_amd as nv
from tests import _gpu as G

pytestmark = pytest.mark.gpu

# 17408 x 5120: 272 super-tiles.  On 256 CUs the cost model picks the wide
# product from 17 columns (32-column shape: 136 workgroups, about 32 us,
# against 45 us for three passes); 24 -> 32-column shape, 48 -> 64-column
# shape, 100 -> 128-column narrow shape (its 136 workgroups fit one round of
# the CUs), 200 -> product shape.
R, K = 17408, 5120
WIDTHS = (24, 48, 100, 200)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load()
    yield
    torch.cuda.synchronize()


def _planes(fmt, W):
    codes = torch.empty(R, K // 2, dtype=torch.uint8, device=G.DEV)
    if fmt == "mxfp4":
        scales = torch.empty(R, K // 32, dtype=torch.uint8, device=G.DEV)
        nv.mxfp4_quantize(W, R, K, 1.0, codes, scales)
        wq, ws = nv.alloc_mx_repacked(R, K, G.DEV)
        nv.mxfp4_repack(codes, scales, R, K, wq, ws)
    else:
        scales = torch.empty(R, K // 16, dtype=torch.uint8, device=G.DEV)
        nv.nvfp4_quantize(W, R, K, 1.0, codes, scales)
        wq, ws = nv.alloc_repacked(R, K, G.DEV)
        nv.nvfp4_repack(codes, scales, R, K, wq, ws)
    return wq, ws


def _gemv(fmt):
    return nv.mxfp4_gemv if fmt == "mxfp4" else nv.nvfp4_gemv


@pytest.fixture(scope="module", params=["nvfp4", "mxfp4"])
def setup(request):
    fmt = request.param
    W = G.seeded_matrix(R, K, 401)
    wq, ws = _planes(fmt, W)
    X = G.seeded_x(max(WIDTHS), K, seed=402)
    return fmt, W, wq, ws, X


def test_shapes_give_the_columns_of_the_widest(setup):
    fmt, W, wq, ws, X = setup
    f = _gemv(fmt)
    wide = max(WIDTHS)
    Y = torch.full((wide, R), float("nan"), dtype=torch.float32, device=G.DEV)
    G.note("wide shapes %s %dx%d n=%d" % (fmt, R, K, wide))
    f(wq, ws, 0.75, R, K, X, wide, Y)
    for n in WIDTHS[:-1]:
        G.note("wide shapes %s %dx%d n=%d" % (fmt, R, K, n))
        y = torch.full((n, R), float("nan"), dtype=torch.float32, device=G.DEV)
        f(wq, ws, 0.75, R, K, X[:n].contiguous(), n, y)
        assert torch.equal(y.view(torch.int32), Y[:n].view(torch.int32)), (fmt, n)
    # the widest against the oracle on sampled rows (every column)
    rows = np.array(sorted({0, 1, 15, 16, 63, 64, 4095, 8191, 12000, 16383, 17343, 17407}))
    Wc = W[torch.as_tensor(rows, device=G.DEV)].cpu().numpy()
    if fmt == "mxfp4":
        c_ref, s_ref = oracle.mx_quantize(Wc, 1.0)
        Y_ref, S = oracle.mx_gemv(c_ref, s_ref, 0.75, G.wl.bf16_bits(X))
    else:
        c_ref, s_ref = oracle.quantize(Wc, 1.0)
        Y_ref, S = oracle.gemv(c_ref, s_ref, 0.75, G.wl.bf16_bits(X))
    G.assert_within_tolerance(Y[:, torch.as_tensor(rows, device=G.DEV)].cpu().numpy(), Y_ref, S,
                              "wide shapes %s sampled rows" % fmt)


@pytest.mark.parametrize("n", WIDTHS[:-1])
def test_shapes_repeat_their_bits(setup, n):
    fmt, W, wq, ws, X = setup
    f = _gemv(fmt)
    x = X[:n].contiguous()
    G.note("wide shapes repeat %s n=%d" % (fmt, n))
    first = torch.empty(n, R, dtype=torch.float32, device=G.DEV)
    f(wq, ws, 1.0, R, K, x, n, first)
    ys = [torch.empty(n, R, dtype=torch.float32, device=G.DEV) for _ in range(4)]
    for i in range(40):
        f(wq, ws, 1.0, R, K, x, n, ys[i % 4])
        if i % 4 == 3:
            torch.cuda.synchronize()
            for y in ys:
                assert torch.equal(y.view(torch.int32), first.view(torch.int32)), (fmt, n, i)


def test_small_matrix_keeps_passes():
    """4096 x 4096 at 24 columns: three passes of the matvec (about 15 us)
    beat the wide product (its 32 workgroups, about 26 us), so every column
    has its one-column bits."""
    r, k, n = 4096, 4096, 24
    W = G.seeded_matrix(r, k, 403)
    codes, scales = G.quantize_gpu(W)
    wq, ws = G.repack_gpu(codes, scales, r, k)
    X = G.seeded_x(n, k, seed=404)
    G.note("passes %dx%d n=%d" % (r, k, n))
    Y = G.gemv_gpu(wq, ws, 1.0, r, k, X)
    for c in (0, 7, 8, 15, 16, 23):
        y1 = G.gemv_gpu(wq, ws, 1.0, r, k, X[c:c + 1].contiguous())
        assert torch.equal(Y[c].view(torch.int32), y1[0].view(torch.int32)), c


@pytest.mark.parametrize("fmt,k", [("nvfp4", 5136), ("mxfp4", 5152)])
def test_shapes_ragged(fmt, k):
    """17401 rows (a partial last super-tile; rows not a multiple of four,
    so the outputs go out one by one) and a partial last octet: 20, 33, 47
    and 97 columns (32-, 64-, 64- and 128-column shapes) equal the same
    columns of a 200-column product bit for bit, which matches the oracle on
    sampled rows, the last ones included."""
    r = 17401
    W = G.seeded_matrix(r, k, 405)
    codes = torch.empty(r, k // 2, dtype=torch.uint8, device=G.DEV)
    if fmt == "mxfp4":
        scales = torch.empty(r, k // 32, dtype=torch.uint8, device=G.DEV)
        nv.mxfp4_quantize(W, r, k, 1.0, codes, scales)
        wq, ws = nv.alloc_mx_repacked(r, k, G.DEV)
        nv.mxfp4_repack(codes, scales, r, k, wq, ws)
    else:
        scales = torch.empty(r, k // 16, dtype=torch.uint8, device=G.DEV)
        nv.nvfp4_quantize(W, r, k, 1.0, codes, scales)
        wq, ws = nv.alloc_repacked(r, k, G.DEV)
        nv.nvfp4_repack(codes, scales, r, k, wq, ws)
    f = _gemv(fmt)
    X = G.seeded_x(200, k, seed=406)
    Y = torch.full((200, r), float("nan"), dtype=torch.float32, device=G.DEV)
    G.note("wide shapes ragged %s %dx%d n=200" % (fmt, r, k))
    f(wq, ws, 1.5, r, k, X, 200, Y)
    for n in (20, 33, 47, 97):
        G.note("wide shapes ragged %s %dx%d n=%d" % (fmt, r, k, n))
        y = torch.full((n, r), float("nan"), dtype=torch.float32, device=G.DEV)
        f(wq, ws, 1.5, r, k, X[:n].contiguous(), n, y)
        assert torch.equal(y.view(torch.int32), Y[:n].view(torch.int32)), (fmt, n)
    rows = np.array([0, 5, 63, 64, 9999, 17343, 17344, 17399, 17400])
    Wc = W[torch.as_tensor(rows, device=G.DEV)].cpu().numpy()
    if fmt == "mxfp4":
        c_ref, s_ref = oracle.mx_quantize(Wc, 1.0)
        Y_ref, S = oracle.mx_gemv(c_ref, s_ref, 1.5, G.wl.bf16_bits(X))
    else:
        c_ref, s_ref = oracle.quantize(Wc, 1.0)
        Y_ref, S = oracle.gemv(c_ref, s_ref, 1.5, G.wl.bf16_bits(X))
    G.assert_within_tolerance(Y[:, torch.as_tensor(rows, device=G.DEV)].cpu().numpy(), Y_ref, S,
                              "wide shapes ragged %s sampled rows" % fmt)
