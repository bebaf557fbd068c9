"""Calls on two streams at once, each with its own outputs and workspace,
give the bits of the same calls made one after another: the library keeps
no state between calls beyond per-device caches filled on first use (the
allocation-free argmax's shared array is the documented exception and is
not used here)."""
import pytest
import torch

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


def _mat(R, K, seed):
    W = G.seeded_matrix(R, K, seed)
    codes, scales = G.quantize_gpu(W)
    return G.repack_gpu(codes, scales, R, K)


def _work(wq, ws, R, K, X, n, outs):
    """One stream's calls: a product, an argmax, a wide product, a batch."""
    y, lg, am, wsp, yw, yb, ab, bw, prods = outs
    nv.nvfp4_gemv(wq, ws, 0.5, R, K, X[:n], n, y)
    nv.nvfp4_gemv_argmax(wq, ws, 0.5, R, K, X[:n], n, lg, am, wsp)
    nv.nvfp4_gemv(wq, ws, 0.5, R, K, X, X.shape[0], yw)
    nv.nvfp4_gemv_batch(prods, K, X[:n], n, bw)


def _outs(wq, ws, R, K, n, nw, wq2, ws2, R2):
    f = lambda *s: torch.full(s, float("nan"), dtype=torch.float32, device=G.DEV)
    i = lambda m: torch.full((m,), -7, dtype=torch.int32, device=G.DEV)
    y, lg, am, yw, yb, ab = f(n, R), f(n, R), i(n), f(nw, R), f(n, R2), i(n)
    wsp = torch.empty(nv.nvfp4_gemv_argmax_workspace_bytes(R, K, n), dtype=torch.uint8, device=G.DEV)
    prods = [dict(wq=wq2, ws=ws2, tscale=1.0, rows=R2, y=yb, argmax=ab), dict(wq=wq, ws=ws, tscale=0.5, rows=R)]
    prods[1]["y"] = f(n, R)
    bw = torch.empty(max(8, nv.nvfp4_gemv_batch_workspace_bytes(prods, K, n)), dtype=torch.uint8, device=G.DEV)
    return [y, lg, am, wsp, yw, yb, ab, bw, prods]


def _results(outs):
    y, lg, am, _, yw, yb, ab, _, prods = outs
    return [t.clone() for t in (y, lg, am, yw, yb, ab, prods[1]["y"])]


def test_two_streams_equal_sequential():
    K, n, nw = 2048, 4, 40
    a, b = _mat(9000, K, 61), _mat(3000, K, 62)
    X0, X1 = G.seeded_x(nw, K, seed=63), G.seeded_x(nw, K, seed=64)
    o0 = _outs(a[0], a[1], 9000, K, n, nw, b[0], b[1], 3000)
    o1 = _outs(b[0], b[1], 3000, K, n, nw, a[0], a[1], 9000)
    G.note("streams: sequential")
    _work(a[0], a[1], 9000, K, X0, n, o0)
    _work(b[0], b[1], 3000, K, X1, n, o1)
    torch.cuda.synchronize()
    ref0, ref1 = _results(o0), _results(o1)
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        for o in (o0, o1):
            for t in (o[0], o[1], o[4], o[5], o[8][1]["y"]):
                t.fill_(float("nan"))
            o[2].fill_(-7)
            o[6].fill_(-7)
        torch.cuda.synchronize()
        G.note("streams: concurrent %d" % rep)
        with torch.cuda.stream(s0):
            _work(a[0], a[1], 9000, K, X0, n, o0)
        with torch.cuda.stream(s1):
            _work(b[0], b[1], 3000, K, X1, n, o1)
        torch.cuda.synchronize()
        for got, want in ((_results(o0), ref0), (_results(o1), ref1)):
            for g_, w_ in zip(got, want):
                assert torch.equal(g_.view(torch.int32), w_.view(torch.int32)), rep


def test_two_streams_split_finish():
    """Two argmax calls whose finish runs split (270000 and 200000 rows of 16
    columns at two columns: 16876 and 12500 keys), on two streams at once,
    each counting on the counter in its own workspace: the rows of the
    sequential calls."""
    K, n = 16, 2
    a, b = _mat(270000, K, 65), _mat(200000, K, 66)
    X0, X1 = G.seeded_x(n, K, seed=67), G.seeded_x(n, K, seed=68)
    am0, am1 = (torch.full((n,), -7, dtype=torch.int32, device=G.DEV) for _ in range(2))
    w0 = torch.full((nv.nvfp4_gemv_argmax_workspace_bytes(270000, K, n),), 0xA5, dtype=torch.uint8, device=G.DEV)
    w1 = torch.full((nv.nvfp4_gemv_argmax_workspace_bytes(200000, K, n),), 0xA5, dtype=torch.uint8, device=G.DEV)
    G.note("streams split finish: sequential")
    nv.nvfp4_gemv_argmax(a[0], a[1], 1.0, 270000, K, X0, n, None, am0, w0)
    nv.nvfp4_gemv_argmax(b[0], b[1], 1.0, 200000, K, X1, n, None, am1, w1)
    torch.cuda.synchronize()
    ref0, ref1 = am0.clone(), am1.clone()
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        am0.fill_(-7)
        am1.fill_(-7)
        torch.cuda.synchronize()
        G.note("streams split finish: concurrent %d" % rep)
        for _ in range(4):
            with torch.cuda.stream(s0):
                nv.nvfp4_gemv_argmax(a[0], a[1], 1.0, 270000, K, X0, n, None, am0, w0)
            with torch.cuda.stream(s1):
                nv.nvfp4_gemv_argmax(b[0], b[1], 1.0, 200000, K, X1, n, None, am1, w1)
        torch.cuda.synchronize()
        assert torch.equal(am0, ref0), rep
        assert torch.equal(am1, ref1), rep
