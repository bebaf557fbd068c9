"""Every entry point captured in one HIP graph gives, on every replay, the
bits of its eager call: the benchmark times graph replays, and the library
must put nothing into a graph that replays differently (no memset nodes, no
state carried between calls).  Between replays the outputs are refilled
with NaN and other eager products run, then the replay's outputs are
compared bit for bit with the eager ones."""
import numpy as np
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


def _nv(R, K, seed):
    W = G.seeded_matrix(R, K, seed)
    codes, scales = G.quantize_gpu(W)
    return G.repack_gpu(codes, scales, R, K)


def _mx(R, K, seed):
    W = G.seeded_matrix(R, K, seed)
    codes = torch.empty(R, K // 2, dtype=torch.uint8, device=G.DEV)
    scales = torch.empty(R, K // 32, dtype=torch.uint8, device=G.DEV)
    nv.mxfp4_quantize(W, R, K, 1.0, codes, scales)
    wq, ws = nv.alloc_mx_repacked(R, K, G.DEV)
    nv.mxfp4_repack(codes, scales, R, K, wq, ws)
    return wq, ws


def _calls():
    """(name, call, outputs): each call writes only its outputs."""
    out = []
    f32 = lambda *s: torch.empty(*s, dtype=torch.float32, device=G.DEV)
    i32 = lambda n: torch.empty(n, dtype=torch.int32, device=G.DEV)
    K = 1024
    X = {n: G.seeded_x(n, K, seed=300 + n) for n in (1, 4, 8, 64)}
    a = _nv(2000, K, 301)
    for n in (1, 4, 8, 64):
        y = f32(n, 2000)
        out.append(("nvfp4_gemv n=%d" % n, lambda y=y, n=n: nv.nvfp4_gemv(a[0], a[1], 0.7, 2000, K, X[n], n, y), [y]))
    b = _nv(9000, K, 302)
    lg, am = f32(4, 9000), i32(4)
    wsp = torch.empty(nv.nvfp4_gemv_argmax_workspace_bytes(9000, K, 4), dtype=torch.uint8, device=G.DEV)
    out.append(("nvfp4_gemv_argmax n=4",
                lambda: nv.nvfp4_gemv_argmax(b[0], b[1], 1.0, 9000, K, X[4], 4, lg, am, wsp), [lg, am]))
    am1 = i32(1)
    out.append(("nvfp4_gemv_argmax_noalloc n=1",
                lambda: nv.nvfp4_gemv_argmax_noalloc(b[0], b[1], 1.0, 9000, K, X[1], 1, None, am1), [am1]))
    F = 1024
    c = _nv(2 * F, K, 303)
    gu, h = f32(1, 2 * F), torch.empty(1, F, dtype=torch.bfloat16, device=G.DEV)
    out.append(("nvfp4_gemv_swiglu", lambda: nv.nvfp4_gemv_swiglu(c[0], c[1], 1.0, K, F, X[1], 1, gu, h), [gu, h]))
    d = _mx(2000, K, 304)
    for n in (1, 64):
        y = f32(n, 2000)
        out.append(("mxfp4_gemv n=%d" % n, lambda y=y, n=n: nv.mxfp4_gemv(d[0], d[1], 1.0, 2000, K, X[n], n, y), [y]))
    yb, lb, ab = f32(4, 2000), f32(4, 9000), i32(4)
    prods = [dict(wq=b[0], ws=b[1], tscale=1.0, rows=9000, y=lb, argmax=ab),
             dict(wq=a[0], ws=a[1], tscale=0.7, rows=2000, y=yb)]
    bw = torch.empty(max(8, nv.nvfp4_gemv_batch_workspace_bytes(prods, K, 4)), dtype=torch.uint8, device=G.DEV)
    out.append(("nvfp4_gemv_batch n=4", lambda: nv.nvfp4_gemv_batch(prods, K, X[4], 4, bw), [yb, lb, ab]))
    # the split argmax finish (more than 12288 keys at two columns, 6144 from
    # three): its counter in the workspace header is zeroed by the product
    # on every replay
    K2 = 16
    X2 = {n: G.seeded_x(n, K2, seed=310 + n) for n in (2, 8)}
    e = _nv(270000, K2, 307)
    for n in (2, 8):
        am_s = i32(n)
        ws_s = torch.empty(nv.nvfp4_gemv_argmax_workspace_bytes(270000, K2, n), dtype=torch.uint8, device=G.DEV)
        out.append(("nvfp4_gemv_argmax split finish n=%d" % n,
                    lambda n=n, am_s=am_s, ws_s=ws_s: nv.nvfp4_gemv_argmax(e[0], e[1], 1.0, 270000, K2, X2[n], n, None,
                                                                           am_s, ws_s), [am_s]))
    am_n = i32(8)
    out.append(("nvfp4_gemv_argmax_noalloc split finish n=8",
                lambda: nv.nvfp4_gemv_argmax_noalloc(e[0], e[1], 1.0, 270000, K2, X2[8], 8, None, am_n), [am_n]))
    f2 = _nv(4000, K2, 308)
    y2, a2 = f32(2, 4000), i32(2)
    prods2 = [dict(wq=e[0], ws=e[1], tscale=1.0, rows=270000, argmax=a2),
              dict(wq=f2[0], ws=f2[1], tscale=1.0, rows=4000, y=y2)]
    bw2 = torch.empty(nv.nvfp4_gemv_batch_workspace_bytes(prods2, K2, 2), dtype=torch.uint8, device=G.DEV)
    out.append(("nvfp4_gemv_batch split finish n=2", lambda: nv.nvfp4_gemv_batch(prods2, K2, X2[2], 2, bw2), [y2, a2]))
    return out


def _bits(t):
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


def test_graph_replays_equal_eager_calls():
    calls = _calls()
    for name, f, outs in calls:
        G.note("eager " + name)
        f()
    torch.cuda.synchronize()
    eager = [[o.clone() for o in outs] for _, _, outs in calls]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _, f, _ in calls:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    G.note("capture")
    with torch.cuda.graph(g):
        for _, f, _ in calls:
            f()
    # eager work between replays: another product into its own buffer
    other = _nv(3000, 1024, 305)
    xo = G.seeded_x(2, 1024, seed=306)
    yo = torch.empty(2, 3000, dtype=torch.float32, device=G.DEV)
    for rep in range(4):
        for _, _, outs in calls:
            for o in outs:
                if o.dtype == torch.int32:
                    o.fill_(-7)
                elif o.dtype == torch.bfloat16:
                    o.view(torch.int16).fill_(-1)
                else:
                    o.fill_(float("nan"))
        nv.nvfp4_gemv(other[0], other[1], 1.0, 3000, 1024, xo, 2, yo)
        torch.cuda.synchronize()
        G.note("replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        for (name, _, outs), ref in zip(calls, eager):
            for o, r in zip(outs, ref):
                assert torch.equal(_bits(o), _bits(r)), "%s differs on replay %d" % (name, rep)
    del g
