"""GPU parity at the full workload sizes, through the same entry points and
launch configuration the benchmark times.  Where the oracle can afford every
output it checks every output; otherwise a fixed sample of rows that covers
the first and last (ragged) tiles.  Quantisation is checked bit-exactly on
the rows the oracle re-quantises itself."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_bit_nvfp4_amd import workloads as wl
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


def _sample_rows(R, count, seed):
    rng = np.random.default_rng(seed)
    rows = set(range(min(16, R))) | set(range(max(0, R - 16), R))
    rows |= set(rng.choice(R, size=min(count, R), replace=False).tolist())
    return np.array(sorted(rows), np.int64)


def _matrix(workload, m, copy=0):
    W = wl.weights(m.rows, m.cols, seed=wl.seed_of(workload.name, m.name, copy),
                   outliers=workload.outliers, device=G.DEV)
    codes, scales = G.quantize_gpu(W, workload.tscale)
    wq, ws = G.repack_gpu(codes, scales, m.rows, m.cols)
    return W, codes, scales, wq, ws


def _oracle_rows(W, codes_gpu, scales_gpu, rows, tscale):
    """Oracle re-quantisation of the sampled rows from the same fp32 weights;
    checks the GPU's codes and scales on those rows bit-exactly."""
    Wr = W[torch.as_tensor(rows, device=W.device)].cpu().numpy()
    c_ref, s_ref = oracle.quantize(Wr, tscale)
    idx = torch.as_tensor(rows, device=codes_gpu.device)
    assert np.array_equal(scales_gpu[idx].cpu().numpy(), s_ref)
    assert np.array_equal(codes_gpu[idx].cpu().numpy(), c_ref)
    return c_ref, s_ref


def test_gemv_256x512_seed0():
    w = wl.WORKLOADS["gemv_256x512"]
    m = w.matrices[0]
    G.note("config gemv_256x512")
    W, codes, scales, wq, ws = _matrix(w, m)
    X = wl.activations(1, m.cols, seed=wl.seed_of(w.name, "x"), device=G.DEV)
    Y = G.gemv_gpu(wq, ws, w.tscale, m.rows, m.cols, X).cpu().numpy()
    c_ref, s_ref = _oracle_rows(W, codes, scales, np.arange(m.rows), w.tscale)
    Y_ref, S = oracle.gemv(c_ref, s_ref, w.tscale, wl.bf16_bits(X))
    G.assert_within_tolerance(Y, Y_ref, S, "gemv_256x512")


@pytest.mark.parametrize("copy", [0, 63])
def test_decode_4096x4096_full(copy):
    w = wl.WORKLOADS["decode_4096x4096"]
    m = w.matrices[0]
    G.note("config decode_4096x4096 copy %d" % copy)
    W, codes, scales, wq, ws = _matrix(w, m, copy)
    X = wl.activations(1, m.cols, seed=wl.seed_of(w.name, "x"), device=G.DEV)
    Y = G.gemv_gpu(wq, ws, w.tscale, m.rows, m.cols, X).cpu().numpy()
    c_ref, s_ref = _oracle_rows(W, codes, scales, np.arange(m.rows), w.tscale)
    Y_ref, S = oracle.gemv(c_ref, s_ref, w.tscale, wl.bf16_bits(X))
    G.assert_within_tolerance(Y, Y_ref, S, "decode_4096x4096")


def test_mlp_27b_decode_layer():
    w = wl.WORKLOADS["mlp_27b_decode"]
    gate_up, down = w.matrices
    X = wl.activations(1, gate_up.cols, seed=wl.seed_of(w.name, "x"), device=G.DEV)
    G.note("config mlp_27b_decode gate_up")
    W1, c1, s1, q1, ss1 = _matrix(w, gate_up)
    gu = G.gemv_gpu(q1, ss1, w.tscale, gate_up.rows, gate_up.cols, X)
    F = down.cols
    rows = _sample_rows(F, 384, 1)
    rows_gu = np.concatenate([rows, rows + F])            # gate row and its up row
    c_ref, s_ref = _oracle_rows(W1, c1, s1, rows_gu, w.tscale)
    Y_ref, S = oracle.gemv_rows(c_ref, s_ref, w.tscale, wl.bf16_bits(X))
    G.assert_within_tolerance(gu.cpu().numpy()[:, rows_gu], Y_ref, S, "mlp gate_up")
    # SwiGLU on the GPU's own gate/up outputs
    h = torch.empty(1, F, dtype=torch.int16, device=G.DEV)
    G.note("config mlp_27b_decode swiglu")
    nv.nvfp4_swiglu(gu, F, 1, h)
    from tests.test_gpu_parity import _check_swiglu
    _check_swiglu(gu.cpu().numpy(), h.cpu().numpy().view(np.uint16))
    # down on the GPU's own bf16 h, every output row
    G.note("config mlp_27b_decode down")
    W2, c2, s2, q2, ss2 = _matrix(w, down)
    hb = h.view(torch.bfloat16)
    y = G.gemv_gpu(q2, ss2, w.tscale, down.rows, down.cols, hb).cpu().numpy()
    c2r, s2r = _oracle_rows(W2, c2, s2, np.arange(down.rows), w.tscale)
    Y2, S2 = oracle.gemv(c2r, s2r, w.tscale, wl.bf16_bits(hb))
    G.assert_within_tolerance(y, Y2, S2, "mlp down")


@pytest.mark.parametrize("name", ["verify_vocab_n4", "verify_vocab_n8"])
def test_verify_vocab_with_full_argmax(name):
    w = wl.WORKLOADS[name]
    mw, head = w.matrices
    n = w.n
    X = wl.activations(n, mw.cols, seed=wl.seed_of(w.name, "x"), device=G.DEV)
    xb = wl.bf16_bits(X)
    G.note("config %s w" % name)
    W1, c1, s1, q1, ss1 = _matrix(w, mw)
    Y1 = G.gemv_gpu(q1, ss1, w.tscale, mw.rows, mw.cols, X).cpu().numpy()
    rows = _sample_rows(mw.rows, 512, 2)
    c_ref, s_ref = _oracle_rows(W1, c1, s1, rows, w.tscale)
    Yr, S = oracle.gemv_rows(c_ref, s_ref, w.tscale, xb)
    G.assert_within_tolerance(Y1[:, rows], Yr, S, "verify w")
    # column identity with N=1 on the same matrix
    for c in range(n):
        y1 = G.gemv_gpu(q1, ss1, w.tscale, mw.rows, mw.cols, X[c:c + 1].contiguous()).cpu().numpy()
        assert np.array_equal(y1[0].view(np.uint32), Y1[c].view(np.uint32))
    del W1
    torch.cuda.empty_cache()
    G.note("config %s lm_head" % name)
    W2, c2, s2, q2, ss2 = _matrix(w, head)
    logits, am = G.gemv_argmax_gpu(q2, ss2, w.tscale, head.rows, head.cols, X)
    W2h = W2.cpu().numpy()
    del W2
    torch.cuda.empty_cache()
    c2r, s2r = oracle.quantize(W2h, w.tscale)             # the oracle's own full quantisation
    del W2h
    assert np.array_equal(c2.cpu().numpy(), c2r)
    assert np.array_equal(s2.cpu().numpy(), s2r)
    Y2, S2 = oracle.gemv(c2r, s2r, w.tscale, xb)
    G.assert_within_tolerance(logits.cpu().numpy(), Y2, S2, "lm_head logits")
    want = oracle.argmax_first(Y2)
    assert list(am.cpu().numpy()) == list(want)
    # the benchmarked launch: both products in one nvfp4_gemv_batch call give
    # the bits of the two calls above
    G.note("config %s batched" % name)
    yb = torch.full((n, mw.rows), float("nan"), dtype=torch.float32, device=G.DEV)
    lb = torch.full((n, head.rows), float("nan"), dtype=torch.float32, device=G.DEV)
    ab = torch.full((n,), -7, dtype=torch.int32, device=G.DEV)
    prods = [dict(wq=q2, ws=ss2, tscale=w.tscale, rows=head.rows, y=lb, argmax=ab),
             dict(wq=q1, ws=ss1, tscale=w.tscale, rows=mw.rows, y=yb)]
    wsp = torch.empty(max(8, nv.nvfp4_gemv_batch_workspace_bytes(prods, mw.cols, n)), dtype=torch.uint8,
                      device=G.DEV)
    nv.nvfp4_gemv_batch(prods, mw.cols, X, n, wsp)
    assert np.array_equal(yb.cpu().numpy().view(np.uint32), Y1.view(np.uint32))
    assert torch.equal(lb.view(torch.int32), logits.view(torch.int32))
    assert list(ab.cpu().numpy()) == list(want)
    # report how far the winner leads the runner-up next to the tolerance
    for c in range(n):
        order = np.argsort(Y2[c])
        margin = Y2[c][order[-1]] - Y2[c][order[-2]]
        bound = 1e-5 * (S2[c][order[-1]] + S2[c][order[-2]]) + 2e-6
        G.note("lm_head column %d: argmax %d, top-2 margin %.4g vs tolerance %.3g" % (
            c, int(want[c]), margin, bound))


def test_prefill_n512_sampled():
    w = wl.WORKLOADS["prefill_n512"]
    m = w.matrices[0]
    G.note("config prefill_n512")
    W, codes, scales, wq, ws = _matrix(w, m)
    X = wl.activations(512, m.cols, seed=wl.seed_of(w.name, "x"), device=G.DEV)
    Y = G.gemv_gpu(wq, ws, w.tscale, m.rows, m.cols, X).cpu().numpy()
    rows = _sample_rows(m.rows, 48, 3)
    c_ref, s_ref = _oracle_rows(W, codes, scales, rows, w.tscale)
    Yr, S = oracle.gemv_rows(c_ref, s_ref, w.tscale, wl.bf16_bits(X))
    G.assert_within_tolerance(Y[:, rows], Yr, S, "prefill n512")


def test_draft_head_8192x4096_full_argmax():
    w = wl.WORKLOADS["draft_head_8192x4096"]
    m = w.matrices[0]
    X = wl.activations(1, m.cols, seed=wl.seed_of(w.name, "x"), device=G.DEV)
    xb = wl.bf16_bits(X)
    for copy in (0, w.copies - 1):
        G.note("config draft_head_8192x4096 copy %d" % copy)
        W, c, s, q, ss = _matrix(w, m, copy)
        logits, am = G.gemv_argmax_gpu(q, ss, w.tscale, m.rows, m.cols, X)
        c_ref, s_ref = oracle.quantize(W.cpu().numpy(), w.tscale)
        assert np.array_equal(c.cpu().numpy(), c_ref)
        assert np.array_equal(s.cpu().numpy(), s_ref)
        Y, S = oracle.gemv(c_ref, s_ref, w.tscale, xb)
        G.assert_within_tolerance(logits.cpu().numpy(), Y, S, "draft head logits")
        assert list(am.cpu().numpy()) == list(oracle.argmax_first(Y))
        # the argmax without stored logits names the same row
        _, am2 = G.gemv_argmax_gpu(q, ss, w.tscale, m.rows, m.cols, X, with_logits=False)
        assert torch.equal(am, am2)


def _mx_matrix(workload, m, copy=0):
    W = wl.weights(m.rows, m.cols, seed=wl.seed_of(workload.name, m.name, copy),
                   outliers=workload.outliers, device=G.DEV)
    codes = torch.empty(m.rows, m.cols // 2, dtype=torch.uint8, device=G.DEV)
    scales = torch.empty(m.rows, m.cols // 32, dtype=torch.uint8, device=G.DEV)
    nv.mxfp4_quantize(W, m.rows, m.cols, workload.tscale, codes, scales)
    wq, ws = nv.alloc_mx_repacked(m.rows, m.cols, G.DEV)
    nv.mxfp4_repack(codes, scales, m.rows, m.cols, wq, ws)
    return W, codes, scales, wq, ws


def test_mxfp4_gemv_17408x5120_full():
    w = wl.WORKLOADS["mxfp4_gemv_17408x5120"]
    m = w.matrices[0]
    X = wl.activations(1, m.cols, seed=wl.seed_of(w.name, "x"), device=G.DEV)
    for copy in (0, w.copies - 1):
        G.note("config mxfp4_gemv_17408x5120 copy %d" % copy)
        W, c, s, q, ss = _mx_matrix(w, m, copy)
        Y = torch.full((1, m.rows), float("nan"), dtype=torch.float32, device=G.DEV)
        nv.mxfp4_gemv(q, ss, w.tscale, m.rows, m.cols, X, 1, Y)
        c_ref, s_ref = oracle.mx_quantize(W.cpu().numpy(), w.tscale)
        assert np.array_equal(c.cpu().numpy(), c_ref)
        assert np.array_equal(s.cpu().numpy(), s_ref)
        Y_ref, S = oracle.mx_gemv(c_ref, s_ref, w.tscale, wl.bf16_bits(X))
        G.assert_within_tolerance(Y.cpu().numpy(), Y_ref, S, "mxfp4 17408x5120")


def test_mxfp4_prefill_n512_sampled():
    w = wl.WORKLOADS["mxfp4_prefill_n512"]
    m = w.matrices[0]
    X = wl.activations(512, m.cols, seed=wl.seed_of(w.name, "x"), device=G.DEV)
    G.note("config mxfp4_prefill_n512")
    W, c, s, q, ss = _mx_matrix(w, m)
    Y = torch.full((512, m.rows), float("nan"), dtype=torch.float32, device=G.DEV)
    nv.mxfp4_gemv(q, ss, w.tscale, m.rows, m.cols, X, 512, Y)
    rows = _sample_rows(m.rows, 256, 5)
    Wr = W[torch.as_tensor(rows, device=W.device)].cpu().numpy()
    c_ref, s_ref = oracle.mx_quantize(Wr, w.tscale)
    idx = torch.as_tensor(rows, device=G.DEV)
    assert np.array_equal(c[idx].cpu().numpy(), c_ref)
    assert np.array_equal(s[idx].cpu().numpy(), s_ref)
    Y_ref, S = oracle.mx_gemv_rows(c_ref, s_ref, w.tscale, wl.bf16_bits(X))
    G.assert_within_tolerance(Y.cpu().numpy()[:, rows], Y_ref, S, "mxfp4 prefill n512")
