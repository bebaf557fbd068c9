"""Every code x scale pair through the products themselves, bit for bit.

The matrices below hold every E2M1 code byte under every scale byte (row r
uses scale byte r mod 256 in all its blocks; element k of a row holds the
codes of byte (k / 2) mod 256).  With X the identity (one-hot columns), the
product's output is one decoded weight:

    Y[c][r] = sum_k w_hat[r][k] X[c][k] = w_hat[r][k_c],

so each product must return RN32(e2m1 * scale * tscale) exactly, the single
rounding the oracle's fp32 target takes.  This proves, on the products'
own instructions, the decode that the dequant export's exhaustive test proves
for that kernel: the matvec's packed E4M3 conversion and E2M1-to-bf16
conversion, the wide kernel's E2M1 conversion, scale multiply and bf16 pack,
and the MXFP4 scale builds, for every scale byte including subnormal,
saturated and NaN ones.  One-hot columns cover all k at n = 1, 4 and 8 (the
matvec), and identity X at n = 512 (the wide contraction); larger tiled
matrices reach the two- and four-tile workgroups, the grouped-load path and
the wide kernel's extra-tile decode.

Comparisons: zeros compare as +0 (a sum that starts at +0 turns a -0 term
into +0), NaN outputs (scale bytes 0x7F and 0xFF) by isnan.  MXFP4 outputs
whose decoded weight e2m1 * 2^(b - 127) lies beyond fp32's range (bytes 253
and 254 with large codes) are outside the products' domain: the sums run in
fp32 before the tensor scale, so the matvec gives the infinity of that sign
there, and the wide product, which decodes to bf16 (the same exponent range),
gives non-finite outputs in those rows.
"""
import numpy as np
import pytest
import torch

import oracle
import block_scaled_bit_nvfp4_amd as nv
from tests import _gpu as G

pytestmark = pytest.mark.gpu

FLT_MAX = float(np.finfo(np.float32).max)
TSCALES = [1.0, 0.37, 2.0 ** -20, 1000.0]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load()
    yield
    torch.cuda.synchronize()


def _table(R, K, mx=False):
    """Canonical codes and scales: row r, scale byte r mod 256 in every block;
    element pair k / 2 of a row holds the code byte (k / 2) mod 256."""
    codes = np.tile((np.arange(K // 2) % 256).astype(np.uint8), (R, 1))
    nb = K // (32 if mx else 16)
    scales = np.tile((np.arange(R) % 256).astype(np.uint8)[:, None], (1, nb))
    return codes, scales


def _planes(codes, scales, R, K, mx):
    cd, sd = G.canonical_to_dev(codes, scales)
    if mx:
        wq, ws = nv.alloc_mx_repacked(R, K, G.DEV)
        nv.mxfp4_repack(cd, sd, R, K, wq, ws)
    else:
        wq, ws = G.repack_gpu(cd, sd, R, K)
    return wq, ws


def _one_hot_products(wq, ws, tscale, R, K, n, mx, ks=None):
    """Y_all[k][r] = product of the n-column call whose column c is e_k, for
    every k (n consecutive k per call; the last call of a ragged k list is
    padded with a repeated k)."""
    ks = np.arange(K) if ks is None else np.asarray(ks)
    eye = torch.zeros(len(ks) + n, K, dtype=torch.bfloat16, device=G.DEV)
    pad = np.concatenate([ks, np.full(n, ks[-1])])
    eye[torch.arange(len(pad), device=G.DEV), torch.as_tensor(pad, device=G.DEV)] = 1.0
    Y = torch.full((len(ks) + n, R), float("nan"), dtype=torch.float32, device=G.DEV)
    f = nv.mxfp4_gemv if mx else nv.nvfp4_gemv
    for i in range(0, len(ks), n):
        f(wq, ws, tscale, R, K, eye[i:i + n], n, Y[i:i + n])
    torch.cuda.synchronize()
    return Y[:len(ks)].cpu().numpy()


def _expected(codes, scales, tscale, mx):
    """RN32 of the exact decoded weight (fp64, oracle), with the one
    documented exception for MXFP4: where e2m1 * 2^(b - 127) itself passes
    fp32's range the fp32 sum is already infinite."""
    if mx:
        with np.errstate(over="ignore", invalid="ignore"):
            w = oracle.mx_dequant(codes, scales, tscale)
            pre = oracle.mx_dequant(codes, scales, 1.0)
            want = w.astype(np.float32)
            over = np.abs(pre) > FLT_MAX
            want[over] = np.where(pre[over] > 0, np.inf, -np.inf).astype(np.float32)
        return want, over
    return oracle.dequant_f32(codes, scales, tscale), np.zeros(codes.shape[:1] + (codes.shape[1] * 2,), bool)


def _assert_bitwise(got, want, what):
    """got, want fp32 [R][K]: equal bits with -0 folded to +0, NaN by isnan."""
    got = got + np.float32(0.0)
    want = want + np.float32(0.0)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "%s: NaN positions differ" % what
    diff = got[~nan].view(np.uint32) != want[~nan].view(np.uint32)
    if diff.any():
        idx = np.argwhere(~nan)[np.nonzero(diff)[0][:5]]
        raise AssertionError("%s: %d of %d outputs differ, e.g. %s" % (
            what, int(diff.sum()), diff.size,
            [(tuple(i), float(got[tuple(i)]), float(want[tuple(i)])) for i in idx]))


# ---------------------------------------------------------------- the matvec

@pytest.mark.parametrize("mx", [False, True], ids=["nvfp4", "mxfp4"])
@pytest.mark.parametrize("n", [1, 4, 8])
@pytest.mark.parametrize("tscale", TSCALES)
def test_matvec_one_hot_every_code_and_scale(mx, n, tscale):
    R, K = 256, 512
    codes, scales = _table(R, K, mx)
    G.note("exhaustive matvec %s n=%d tscale=%g" % ("mxfp4" if mx else "nvfp4", n, tscale))
    wq, ws = _planes(codes, scales, R, K, mx)
    got = _one_hot_products(wq, ws, tscale, R, K, n, mx).T
    want, _ = _expected(codes, scales, tscale, mx)
    nan = np.isnan(want)
    assert nan.sum() == (1 if mx else 2) * K          # NaN scale bytes: 0xFF (E8M0); 0x7F, 0xFF (E4M3)
    _assert_bitwise(got, want, "matvec n=%d" % n)


@pytest.mark.parametrize("mx", [False, True], ids=["nvfp4", "mxfp4"])
@pytest.mark.parametrize("R,K,n", [
    # 288 tiles of 36-octet rows: two tiles per workgroup, eight waves of four
    # or five octets; at n = 1 the grouped activation/scale loads
    (4608, 4608, 1), (4608, 4608, 8),
    # 4112 tiles: two tiles per workgroup, four past four columns (NVFP4)
    (65792, 512, 1), (65792, 512, 6),
])
def test_matvec_one_hot_multi_tile(mx, R, K, n):
    codes, scales = _table(R, K, mx)
    G.note("exhaustive matvec multi-tile %s %dx%d n=%d" % ("mxfp4" if mx else "nvfp4", R, K, n))
    wq, ws = _planes(codes, scales, R, K, mx)
    got = _one_hot_products(wq, ws, 0.37, R, K, n, mx).T
    want, _ = _expected(codes, scales, 0.37, mx)
    _assert_bitwise(got, want, "matvec %dx%d n=%d" % (R, K, n))


# ------------------------------------------------------ the wide contraction

@pytest.mark.parametrize("mx", [False, True], ids=["nvfp4", "mxfp4"])
@pytest.mark.parametrize("tscale", TSCALES)
def test_wide_identity_every_code_and_scale(mx, tscale):
    """X = the 512 x 512 identity at n = 512: Y[c][r] = w_hat[r][c].  17408
    rows (272 super-tiles) make the kernel cut its row groups to whole CU
    rounds and hand the 64 remaining tiles to the workgroups as extra tiles,
    so both decode sites run."""
    R, K, n = 17408, 512, 512
    codes, scales = _table(R, K, mx)
    G.note("exhaustive wide %s tscale=%g" % ("mxfp4" if mx else "nvfp4", tscale))
    wq, ws = _planes(codes, scales, R, K, mx)
    X = torch.eye(n, K, dtype=torch.bfloat16, device=G.DEV)
    Y = torch.full((n, R), float("nan"), dtype=torch.float32, device=G.DEV)
    (nv.mxfp4_gemv if mx else nv.nvfp4_gemv)(wq, ws, tscale, R, K, X, n, Y)
    got = Y.cpu().numpy().T
    want, over = _expected(codes, scales, tscale, mx)
    if mx:
        # rows holding a weight beyond bf16's (= fp32's) range decode to an
        # infinity, and inf * 0 makes their other outputs NaN
        bad_rows = over.any(axis=1)
        assert sorted(set((np.nonzero(bad_rows)[0] % 256).tolist())) == [253, 254]
        assert not np.isfinite(got[bad_rows]).any()
        got, want = got[~bad_rows], want[~bad_rows]
    _assert_bitwise(got, want, "wide n=512")
