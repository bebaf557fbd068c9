"""A seeded sweep of random shapes against the oracle: rows from 1 to about
70000 (ragged tiles and super-tiles), columns any multiple of 16 (32 for
MXFP4; ragged octets), every n up to 8 plus some wide n, four tensor
scales, both formats.  Each case checks the product within the parity
tolerance, and for NVFP4 at n <= 8 the argmax and the batched call.

The argmax must equal the argmax of the GPU's own logits (lowest index on
ties) and the oracle's, except where the oracle's two leading values lie
within the parity tolerance of each other: there either index is a correct
answer at fp32 (the configured workloads are checked for identity
elsewhere).

A second sweep takes wide n (9 to 600: the passes of the matvec and every
workgroup shape of the MFMA contraction, as the cost model picks them) on
ragged rows and rows of any whole number of blocks, checks every column on
sampled rows against the oracle, and requires a second call to repeat the
bits."""
import numpy as np
import pytest
import torch

import oracle
import block_scaled_bit_nvfp4_amd as nv
from tests import _gpu as G

pytestmark = pytest.mark.gpu

TSCALES = [1.0, 0.37, 3.0, 2.0 ** -10]


def _cases(count=28, large=10, seed=2024):
    """count shapes log-uniform over rows and columns, then `large` with
    both dimensions in the thousands (several super-tiles of long rows)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count + large):
        mx = i % 4 == 3
        step = 32 if mx else 16
        if i < count:
            R = int(np.exp(rng.uniform(0, np.log(70000))))
            K = step * max(1, int(np.exp(rng.uniform(0, np.log(20000 / step)))))
        else:
            R = int(rng.integers(2000, 12001))
            K = step * int(rng.integers(2000 // step, 6000 // step + 1))
        while R * K > 24_000_000:
            R = max(1, R // 2)
        n = int(rng.integers(1, 9)) if rng.random() < 0.8 else int(rng.integers(9, 41))
        out.append((R, K, n, TSCALES[(i // 4 + i) % 4], mx, 9000 + i))
    return out


CASES = _cases()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load()
    yield
    torch.cuda.synchronize()


def _prepare(R, K, seed, tscale, mx):
    W = G.seeded_matrix(R, K, seed)
    if mx:
        codes = torch.empty(R, K // 2, dtype=torch.uint8, device=G.DEV)
        scales = torch.empty(R, K // 32, dtype=torch.uint8, device=G.DEV)
        nv.mxfp4_quantize(W, R, K, tscale, codes, scales)
        wq, ws = nv.alloc_mx_repacked(R, K, G.DEV)
        nv.mxfp4_repack(codes, scales, R, K, wq, ws)
        c_ref, s_ref = oracle.mx_quantize(W.cpu().numpy(), tscale)
    else:
        codes, scales = G.quantize_gpu(W, tscale)
        wq, ws = G.repack_gpu(codes, scales, R, K)
        c_ref, s_ref = oracle.quantize(W.cpu().numpy(), tscale)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    return wq, ws, c_ref, s_ref


def _check_argmax(am, logits, Y_ref, S, what):
    own = np.argmax(logits, axis=1)
    assert list(am) == list(own), what + ": argmax is not that of the logits"
    want = oracle.argmax_first(Y_ref)
    tol = oracle.tolerance(S)
    for c in range(Y_ref.shape[0]):
        if am[c] != want[c]:
            a, b = int(am[c]), int(want[c])
            gap = abs(Y_ref[c, a] - Y_ref[c, b])
            assert gap <= tol[c, a] + tol[c, b], "%s column %d: %d against the oracle's %d" % (what, c, a, b)


@pytest.mark.parametrize("R,K,n,tscale,mx,seed", CASES,
                         ids=["%s-%dx%d-n%d" % ("mx" if c[4] else "nv", c[0], c[1], c[2]) for c in CASES])
def test_random_shape(R, K, n, tscale, mx, seed):
    what = "%s %dx%d n=%d tscale=%g" % ("mxfp4" if mx else "nvfp4", R, K, n, tscale)
    G.note("random " + what)
    wq, ws, c_ref, s_ref = _prepare(R, K, seed, tscale, mx)
    X = G.seeded_x(n, K, seed=seed + 1)
    Y = torch.full((n, R), float("nan"), dtype=torch.float32, device=G.DEV)
    (nv.mxfp4_gemv if mx else nv.nvfp4_gemv)(wq, ws, tscale, R, K, X, n, Y)
    Y_ref, S = (oracle.mx_gemv if mx else oracle.gemv)(c_ref, s_ref, tscale, G.wl.bf16_bits(X))
    y = Y.cpu().numpy()
    G.assert_within_tolerance(y, Y_ref, S, what)
    if mx or n > 8:
        return
    logits, am = G.gemv_argmax_gpu(wq, ws, tscale, R, K, X)
    assert torch.equal(logits.view(torch.int32), Y.view(torch.int32)), what + ": argmax logits"
    _check_argmax(am.cpu().numpy(), y, Y_ref, S, what)
    # the same product in a batch beside a second one of the same columns
    R2 = max(1, (R * 3) // 5 + 7)
    wq2, ws2, _, _ = _prepare(R2, K, seed + 2, 1.0, False)
    y1 = torch.full((n, R), float("nan"), dtype=torch.float32, device=G.DEV)
    a1 = torch.full((n,), -7, dtype=torch.int32, device=G.DEV)
    y2 = torch.full((n, R2), float("nan"), dtype=torch.float32, device=G.DEV)
    prods = [dict(wq=wq, ws=ws, tscale=tscale, rows=R, y=y1, argmax=a1),
             dict(wq=wq2, ws=ws2, tscale=1.0, rows=R2, y=y2)]
    wsp = torch.full((max(8, nv.nvfp4_gemv_batch_workspace_bytes(prods, K, n)),), 0xA5, dtype=torch.uint8,
                     device=G.DEV)
    nv.nvfp4_gemv_batch(prods, K, X, n, wsp)
    assert torch.equal(y1.view(torch.int32), Y.view(torch.int32)), what + ": batched product"
    assert torch.equal(a1, am), what + ": batched argmax"
    assert torch.equal(y2.view(torch.int32), G.gemv_gpu(wq2, ws2, 1.0, R2, K, X).view(torch.int32)), \
        what + ": batched second product"


def _wide_cases(count=44, seed=777):
    """Rows log-uniform over 20..60000, columns over 2..12000 blocks, n from
    one of four ranges (9..32, 33..64, 65..128, 129..600), both formats."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        mx = i % 3 == 2
        step = 32 if mx else 16
        R = int(np.exp(rng.uniform(np.log(20), np.log(60000))))
        K = step * max(1, int(np.exp(rng.uniform(np.log(2), np.log(12000 / step)))))
        n = int(rng.choice([int(rng.integers(9, 33)), int(rng.integers(33, 65)), int(rng.integers(65, 129)),
                            int(rng.integers(129, 601))]))
        while R * K > 40_000_000:
            R = max(1, R // 2)
        out.append((R, K, n, TSCALES[i % 4], mx, 5000 + i))
    return out


WIDE_CASES = _wide_cases()


@pytest.mark.parametrize("R,K,n,tscale,mx,seed", WIDE_CASES,
                         ids=["%s-%dx%d-n%d" % ("mx" if c[4] else "nv", c[0], c[1], c[2]) for c in WIDE_CASES])
def test_random_wide_shape(R, K, n, tscale, mx, seed):
    what = "%s %dx%d n=%d tscale=%g" % ("mxfp4" if mx else "nvfp4", R, K, n, tscale)
    G.note("random wide " + what)
    W = G.seeded_matrix(R, K, seed)
    codes = torch.empty(R, K // 2, dtype=torch.uint8, device=G.DEV)
    if mx:
        scales = torch.empty(R, K // 32, dtype=torch.uint8, device=G.DEV)
        nv.mxfp4_quantize(W, R, K, tscale, codes, scales)
        wq, ws = nv.alloc_mx_repacked(R, K, G.DEV)
        nv.mxfp4_repack(codes, scales, R, K, wq, ws)
    else:
        codes, scales = G.quantize_gpu(W, tscale)
        wq, ws = G.repack_gpu(codes, scales, R, K)
    f = nv.mxfp4_gemv if mx else nv.nvfp4_gemv
    X = G.seeded_x(n, K, seed=seed + 1)
    Y = torch.full((n, R), float("nan"), dtype=torch.float32, device=G.DEV)
    f(wq, ws, tscale, R, K, X, n, Y)
    Y2 = torch.full((n, R), float("nan"), dtype=torch.float32, device=G.DEV)
    f(wq, ws, tscale, R, K, X, n, Y2)
    assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32)), what + ": a second call differs"
    rng = np.random.default_rng(seed)
    rows = np.array(sorted(set([0, R // 2, R - 1] + [int(r) for r in rng.integers(0, R, size=min(R, 24))])))
    sel = torch.as_tensor(rows, device=G.DEV)
    Wc = W[sel].cpu().numpy()
    if mx:
        c_ref, s_ref = oracle.mx_quantize(Wc, tscale)
        Y_ref, S = oracle.mx_gemv(c_ref, s_ref, tscale, G.wl.bf16_bits(X))
    else:
        c_ref, s_ref = oracle.quantize(Wc, tscale)
        Y_ref, S = oracle.gemv(c_ref, s_ref, tscale, G.wl.bf16_bits(X))
    G.assert_within_tolerance(Y[:, sel].cpu().numpy(), Y_ref, S, what + " (sampled rows)")
