"""nvfp4_gemv_batch: several products of one X in one launch give, product by
product, the bits of their own nvfp4_gemv / nvfp4_gemv_argmax calls, on the
fused path (one product launch) and on the per-product fallback, and the
argmax rows equal the oracle's."""
import numpy as np
import pytest
import torch

import oracle
import block_scaled_bit_nvfp4_amd as nv
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load()
    yield
    torch.cuda.synchronize()


def _matrix(R, K, seed):
    W = G.seeded_matrix(R, K, seed)
    codes, scales = G.quantize_gpu(W)
    wq, ws = G.repack_gpu(codes, scales, R, K)
    return W, wq, ws


def _run(shapes, K, n, seed, with_y=True):
    """shapes: list of (rows, argmax?); returns per product (y, argmax) of the
    batch and of the single calls, and the matrices."""
    mats = [_matrix(R, K, seed + i) for i, (R, _) in enumerate(shapes)]
    X = G.seeded_x(n, K, seed=seed + 100)
    prods = []
    for (R, am), (_, wq, ws) in zip(shapes, mats):
        y = torch.full((n, R), float("nan"), dtype=torch.float32, device=G.DEV) if (with_y or not am) else None
        a = torch.full((n,), -7, dtype=torch.int32, device=G.DEV) if am else None
        prods.append(dict(wq=wq, ws=ws, tscale=0.75, rows=R, y=y, argmax=a))
    nbytes = nv.nvfp4_gemv_batch_workspace_bytes(prods, K, n)
    wsp = torch.full((max(nbytes, 8),), 0xA5, dtype=torch.uint8, device=G.DEV)
    G.note("batch %s K=%d n=%d" % (shapes, K, n))
    nv.nvfp4_gemv_batch(prods, K, X, n, wsp)
    singles = []
    for (R, am), (_, wq, ws) in zip(shapes, mats):
        if am:
            singles.append(G.gemv_argmax_gpu(wq, ws, 0.75, R, K, X))
        else:
            singles.append((G.gemv_gpu(wq, ws, 0.75, R, K, X), None))
    return prods, singles, mats, X


def _same(prods, singles):
    for i, (p, (y, a)) in enumerate(zip(prods, singles)):
        if p["y"] is not None:
            assert torch.equal(p["y"].view(torch.int32), y.view(torch.int32)), i
        if p["argmax"] is not None:
            assert torch.equal(p["argmax"], a), i


@pytest.mark.parametrize("n", [4, 8])
def test_verify_pair_one_launch_equals_single_calls(n):
    """The 151936 x 5120 vocabulary head with its argmax and the 17408 x 5120
    matrix: both split a row over eight waves, so one launch, at the head's
    two (n = 4) or four (n = 8) tiles per workgroup."""
    prods, singles, _, _ = _run([(151936, True), (17408, False)], 5120, n, seed=40)
    _same(prods, singles)


@pytest.mark.parametrize("shapes,K,n", [
    # one launch: three products of one tile per workgroup, eight waves a row
    ([(2000, True), (700, False), (4176, True)], 1024, 1),
    # one launch at two tiles per workgroup, where the 9000-row product alone
    # takes one (grouped one-column loads)
    ([(70000, False), (9000, True)], 2048, 1),
    # one launch at four tiles per workgroup (five waves a row) for a product
    # that alone takes one
    ([(65620, False), (1040, True)], 528, 5),
    # four products of single-octet rows
    ([(300, True), (300, True), (17, False), (129, True)], 96, 8),
    # eight against sixteen waves a row: each product's own launch
    ([(9000, False), (700, True)], 2048, 3),
    # a batch of one
    ([(1024, True)], 512, 2),
])
def test_batch_equals_single_calls(shapes, K, n):
    prods, singles, mats, X = _run(shapes, K, n, seed=41 + n)
    _same(prods, singles)
    for (R, am), p, (W, _, _) in zip(shapes, prods, mats):
        if am:
            c, s = oracle.quantize(W.cpu().numpy())
            Y_ref, _ = oracle.gemv(c, s, 0.75, G.wl.bf16_bits(X))
            assert list(p["argmax"].cpu().numpy()) == list(oracle.argmax_first(Y_ref))


def test_batch_argmax_without_logits():
    prods, singles, _, _ = _run([(2000, True), (3000, True)], 1024, 4, seed=50, with_y=False)
    for p, (_, a) in zip(prods, singles):
        assert p["y"] is None
        assert torch.equal(p["argmax"], a)
