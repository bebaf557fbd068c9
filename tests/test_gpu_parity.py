"""GPU parity of the HIP library against the fp64 CPU oracle at sizes the
oracle finishes in seconds (several tiles and steps, ragged tails), through
the C ABI.  Bit-exact: quantise, repack, dequant, argmax.  Tolerance
|y - y_ref| <= 1e-5 * sum|w*x| + 1e-6: the products."""
import math

import numpy as np
import pytest
import torch

import oracle
import block_scaled_bit_nvfp4_amd as nv
from tests import _gpu as G
from tests.conftest import golden_lines

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_bit_nvfp4_amd as nv
    nv.load()                       # fails loudly if the HIP library is missing
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------ decode, exact

def _all_codes_all_scales():
    """256 rows x 512 cols: row r uses scale byte r in every block and holds
    every code byte 0..255 once, so every (code, scale) pair appears."""
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    scales = np.tile(np.arange(256, dtype=np.uint8)[:, None], (1, 32))
    return codes, scales


@pytest.mark.parametrize("tscale", [1.0, 0.37, 2.0**-20, 1000.0])
def test_dequant_exhaustive_code_scale_table(tscale):
    codes, scales = _all_codes_all_scales()
    R, K = 256, 512
    G.note("dequant exhaustive tscale=%g" % tscale)
    cd, sd = G.canonical_to_dev(codes, scales)
    wq, ws = G.repack_gpu(cd, sd, R, K)
    f32 = torch.empty(R, K, dtype=torch.float32, device=G.DEV)
    b16 = torch.empty(R, K, dtype=torch.int16, device=G.DEV)
    import block_scaled_bit_nvfp4_amd as nv
    nv.nvfp4_dequant(wq, ws, tscale, R, K, f32, b16)
    got32 = f32.cpu().numpy()
    got16 = b16.cpu().numpy().view(np.uint16)
    want32 = oracle.dequant_f32(codes, scales, tscale)
    want16 = oracle.dequant_bf16_bits(codes, scales)
    nan = np.isnan(want32)
    assert nan.sum() == 2 * 512
    assert np.array_equal(np.isnan(got32), nan)
    assert np.array_equal(got32[~nan].view(np.uint32), want32[~nan].view(np.uint32))
    g16 = (got16.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(np.isnan(g16), nan)
    assert np.array_equal(got16[~nan], want16[~nan])


# ---------------------------------------------------------- quantise, exact

def test_quantize_hand_worked_blocks():
    for line in golden_lines("quantize_blocks.txt"):
        ts, ws_, sb, cb = [p.strip() for p in line.split("|")]
        W = torch.tensor([[float(x) for x in ws_.split()]], dtype=torch.float32, device=G.DEV)
        G.note("quantize golden block tscale=%s" % ts)
        codes, scales = G.quantize_gpu(W, float(ts))
        assert scales.cpu().numpy()[0, 0] == int(sb, 16), line
        assert list(codes.cpu().numpy()[0]) == [int(x, 16) for x in cb.split()], line


@pytest.mark.parametrize("R,K,seed,outliers,tscale", [
    (256, 512, 0, False, 1.0),
    (33, 1040, 1, True, 1.0),
    (100, 2048, 2, True, 0.01),
    (7, 16, 3, True, 3.0),
])
def test_quantize_bitexact(R, K, seed, outliers, tscale):
    W = G.seeded_matrix(R, K, seed, outliers)
    W[0, :16] *= 1e5                      # a saturated-scale block
    W[-1, 16 % K:32 if K >= 32 else 16] = 0.0
    G.note("quantize %dx%d seed %d" % (R, K, seed))
    codes, scales = G.quantize_gpu(W, tscale)
    c_ref, s_ref = oracle.quantize(W.cpu().numpy(), tscale)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)


def test_quantize_exact_ties_and_signed_zero():
    ties = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    g = torch.Generator().manual_seed(4)
    W = ties[torch.randint(0, 8, (16, 256), generator=g)] * (torch.randint(0, 2, (16, 256), generator=g) * 2 - 1)
    W[:, ::16] = 6.0
    W = W * 2.0**-5
    W[3, 5] = -0.0
    W = W.to(torch.float32).to(G.DEV)
    G.note("quantize ties")
    codes, scales = G.quantize_gpu(W)
    c_ref, s_ref = oracle.quantize(W.cpu().numpy())
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)


# ------------------------------------------------------------ repack, exact

@pytest.mark.parametrize("R,K", [(17, 32), (16, 1024), (33, 1040), (1, 16), (50, 2064), (256, 512)])
def test_repack_bytes_equal_reference(R, K):
    rng = np.random.default_rng(R * 7 + K)
    codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (R, K // 16), dtype=np.uint8)
    G.note("repack %dx%d" % (R, K))
    cd, sd = G.canonical_to_dev(codes, scales)
    wq, ws = G.repack_gpu(cd, sd, R, K)
    rq, rs = oracle.repack(codes, scales)
    assert np.array_equal(wq.cpu().numpy(), rq)
    assert np.array_equal(ws.cpu().numpy(), rs)


# --------------------------------------------------------- products, tolerance

def _prepare(R, K, seed, outliers=True, tscale=1.0):
    W = G.seeded_matrix(R, K, seed, outliers)
    codes, scales = G.quantize_gpu(W, tscale)
    wq, ws = G.repack_gpu(codes, scales, R, K)
    c_ref, s_ref = oracle.quantize(W.cpu().numpy(), tscale)
    return wq, ws, c_ref, s_ref


@pytest.mark.parametrize("R,K,n,tscale", [
    (256, 512, 1, 1.0),        # the 256 x 512 single matvec, seed 0 weights
    (100, 2064, 1, 1.0),       # ragged rows, a partial last step
    (48, 3072, 2, 0.5),
    (129, 4096, 3, 1.0),
    (64, 5120, 4, 1.0),
    (40, 1024, 5, 2.0),
    (23, 1088, 6, 1.0),
    (31, 96, 7, 1.0),
    (300, 17408, 8, 1.0),
    (16, 16, 1, 1.0),          # a single block
    # two tiles per workgroup (257..512 tiles with rows over 32 octets, or
    # over 4096 tiles), a ragged last octet and wave octet ranges that are no
    # multiple of four: n = 1 takes the grouped activation/scale loads
    (4176, 4112, 1, 1.0),
    (4176, 4112, 2, 1.0),
    (65600, 528, 1, 0.5),
    # past four columns the tiles per workgroup double: two for 261 tiles of
    # 17-octet rows and for 563 tiles, four for 4102 tiles (ragged rows)
    (4176, 2064, 7, 1.0),
    (9000, 1040, 6, 1.0),
    (65620, 528, 5, 1.0),
    (65600, 528, 8, 0.5),
])
def test_gemv_parity(R, K, n, tscale):
    seed = 0 if (R, K) == (256, 512) else R + K
    wq, ws, c_ref, s_ref = _prepare(R, K, seed, outliers=(R, K) != (256, 512), tscale=tscale)
    X = G.seeded_x(n, K, seed=seed + 1)
    G.note("gemv %dx%d n=%d" % (R, K, n))
    Y = G.gemv_gpu(wq, ws, tscale, R, K, X).cpu().numpy()
    Y_ref, S = oracle.gemv(c_ref, s_ref, tscale, G.wl.bf16_bits(X))
    G.assert_within_tolerance(Y, Y_ref, S, "gemv %dx%d n=%d" % (R, K, n))


@pytest.mark.parametrize("R,K,n", [
    (80, 1024, 12), (80, 1024, 33),
    (1000, 1040, 130),     # ragged rows, a partial k chunk, two column tiles
    (257, 2064, 9),        # one row past a tile, K not a multiple of 64
    (17, 16, 300),         # a single block per row
    (4096, 512, 256),      # several workgroups of full tiles
])
def test_gemv_wide_parity(R, K, n):
    wq, ws, c_ref, s_ref = _prepare(R, K, 77 + R + K)
    X = G.seeded_x(n, K, seed=78 + n)
    G.note("gemv wide %dx%d n=%d" % (R, K, n))
    Y = G.gemv_gpu(wq, ws, 1.0, R, K, X).cpu().numpy()
    Y_ref, S = oracle.gemv(c_ref, s_ref, 1.0, G.wl.bf16_bits(X))
    G.assert_within_tolerance(Y, Y_ref, S, "gemv wide %dx%d n=%d" % (R, K, n))


def test_gemv_exact_special_cases():
    R, K = 64, 2048
    wq, ws, c_ref, s_ref = _prepare(R, K, 5)
    w_hat32 = oracle.dequant_f32(c_ref, s_ref, 1.0)
    # one-hot x: y[r] is w_hat[r][k] rounded to fp32, bit for bit (a sum whose
    # other terms are +0 turns a -0 term into +0, so zeros compare as +0)
    w_hat32 = w_hat32 + np.float32(0.0)
    for k in (0, 1, 17, 1000, 2047):
        x = torch.zeros(1, K, dtype=torch.bfloat16, device=G.DEV)
        x[0, k] = 1.0
        G.note("gemv one-hot k=%d" % k)
        y = G.gemv_gpu(wq, ws, 1.0, R, K, x).cpu().numpy()[0]
        assert np.array_equal(y.view(np.uint32), w_hat32[:, k].view(np.uint32)), k
    X = G.seeded_x(1, K, seed=6)
    y = G.gemv_gpu(wq, ws, 1.0, R, K, X)
    # x = 0 -> 0; x -> -x flips every bit of sign only; tscale * 2^j scales exactly
    z = G.gemv_gpu(wq, ws, 1.0, R, K, torch.zeros_like(X))
    assert torch.count_nonzero(z).item() == 0
    yn = G.gemv_gpu(wq, ws, 1.0, R, K, -X)
    assert torch.equal(yn, -y)
    for j in (-3, 5):
        yj = G.gemv_gpu(wq, ws, 2.0**j, R, K, X)
        assert torch.equal(yj, y * 2.0**j)


@pytest.mark.parametrize("R,K", [
    (1040, 5120),
    # shapes whose tiles per workgroup change with the column count: 261
    # tiles of 17-octet rows and 563 tiles (one tile, two past four
    # columns), 4102 tiles (two tiles, four past four columns)
    (4176, 2064), (9000, 1040), (65620, 528),
])
def test_gemv_deterministic_and_column_identity(R, K):
    """Every width n = 1..8 gives, in column c, the bits of the one-column
    product of X[c] (the slots, lanes and summation order of a column do not
    depend on n), and the same bits again on a second launch.  The argmax
    form at every width gives those logits and, per column, the row the
    one-column argmax names."""
    wq, ws, _, _ = _prepare(R, K, 9)
    X = G.seeded_x(8, K, seed=10)
    singles, single_am = [], []
    for c in range(8):
        G.note("column identity %dx%d single column %d" % (R, K, c))
        singles.append(G.gemv_gpu(wq, ws, 1.0, R, K, X[c:c + 1].contiguous()))
        lg, am = G.gemv_argmax_gpu(wq, ws, 1.0, R, K, X[c:c + 1].contiguous())
        assert torch.equal(lg.view(torch.int32), singles[c].view(torch.int32)), c
        single_am.append(int(am.item()))
    for n in range(1, 9):
        G.note("column identity %dx%d n=%d" % (R, K, n))
        Xn = X[:n].contiguous()
        y = G.gemv_gpu(wq, ws, 1.0, R, K, Xn)
        again = G.gemv_gpu(wq, ws, 1.0, R, K, Xn)
        assert torch.equal(y.view(torch.int32), again.view(torch.int32)), n
        logits, am = G.gemv_argmax_gpu(wq, ws, 1.0, R, K, Xn)
        assert torch.equal(logits.view(torch.int32), y.view(torch.int32)), n
        for c in range(n):
            assert torch.equal(y[c].view(torch.int32), singles[c][0].view(torch.int32)), (c, n)
        assert [int(v) for v in am.cpu().numpy()] == single_am[:n], n


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("R,K,widths", [
    (17408, 5120, (9, 16)),             # two passes beat the wide product; from 17 columns it wins
    (4096, 4096, (9, 17, 24, 32, 40)),  # the wide product's 32 workgroups: passes to 40 columns
    (1000, 2080, (9, 12, 16, 32)),      # ragged rows and octets
])
def test_matvec_passes_column_identity(fmt, R, K, widths):
    """9..128 columns run as passes of the matvec where the cost model
    estimates them faster than the wide product (on 256 CUs: 17408 x 5120 to
    16 columns, 4096 x 4096 to 40, 1000 x 2080 past 32): column c then has
    the bits of the one-column product of X[c], and every output is within
    the parity tolerance of the oracle."""
    mx = fmt == "mxfp4"
    W = G.seeded_matrix(R, K, 31)
    if mx:
        codes = torch.empty(R, K // 2, dtype=torch.uint8, device=G.DEV)
        scales = torch.empty(R, K // 32, dtype=torch.uint8, device=G.DEV)
        nv.mxfp4_quantize(W, R, K, 1.0, codes, scales)
        wq, ws = nv.alloc_mx_repacked(R, K, G.DEV)
        nv.mxfp4_repack(codes, scales, R, K, wq, ws)
        c_ref, s_ref = oracle.mx_quantize(W.cpu().numpy(), 1.0)
    else:
        wq, ws, c_ref, s_ref = _prepare(R, K, 31)
    f = nv.mxfp4_gemv if mx else nv.nvfp4_gemv
    cols = max(widths)
    X = G.seeded_x(cols, K, seed=32)
    singles = torch.full((cols, R), float("nan"), dtype=torch.float32, device=G.DEV)
    for c in range(cols):
        f(wq, ws, 0.5, R, K, X[c:c + 1].contiguous(), 1, singles[c:c + 1])
    for n in widths:
        G.note("passes %s %dx%d n=%d" % (fmt, R, K, n))
        y = torch.full((n, R), float("nan"), dtype=torch.float32, device=G.DEV)
        f(wq, ws, 0.5, R, K, X[:n].contiguous(), n, y)
        assert torch.equal(y.view(torch.int32), singles[:n].view(torch.int32)), n
    Y_ref, S = (oracle.mx_gemv if mx else oracle.gemv)(c_ref, s_ref, 0.5, G.wl.bf16_bits(X[:16]))
    G.assert_within_tolerance(singles[:16].cpu().numpy(), Y_ref, S, "passes %s %dx%d" % (fmt, R, K))


# -------------------------------------------------------------- argmax, exact

@pytest.mark.parametrize("R,K,n", [
    (2000, 1024, 1), (2000, 1024, 4), (2000, 1024, 8),
    # two and four tiles per workgroup past four columns
    (9000, 1040, 6), (65620, 528, 5),
    # either side of the split finish's thresholds: 12288 keys at one or two
    # columns, 6144 from three
    (393216, 16, 1), (393280, 16, 1), (32768, 16, 3), (32832, 16, 3),
    # one workgroup, 8438 keys in one pass; the split finish (16 workgroups):
    # one pass over each workgroup's share at 270000 rows, two at 600000
    (270000, 16, 1), (270000, 16, 5), (270000, 16, 8), (600000, 16, 1), (600000, 16, 8),
])
def test_argmax_matches_oracle(R, K, n):
    wq, ws, c_ref, s_ref = _prepare(R, K, 11 + n + (0 if R == 2000 else R))
    X = G.seeded_x(n, K, seed=12)
    G.note("argmax %dx%d n=%d" % (R, K, n))
    logits, am = G.gemv_argmax_gpu(wq, ws, 1.0, R, K, X)
    Y_ref, S = oracle.gemv(c_ref, s_ref, 1.0, G.wl.bf16_bits(X))
    G.assert_within_tolerance(logits.cpu().numpy(), Y_ref, S, "argmax logits")
    assert list(am.cpu().numpy()) == list(oracle.argmax_first(Y_ref))
    # logits are the same bits as the plain product
    y = G.gemv_gpu(wq, ws, 1.0, R, K, X)
    assert torch.equal(y.view(torch.int32), logits.view(torch.int32))
    _, am2 = G.gemv_argmax_gpu(wq, ws, 1.0, R, K, X, with_logits=False)
    assert torch.equal(am, am2)


def test_argmax_workspace_reused_across_calls():
    """One workspace of garbage bytes, sized for the largest call, serves
    back-to-back calls of different inputs and shapes."""
    import block_scaled_bit_nvfp4_amd as nv
    # one-workgroup and split finishes in turn: the split one's counter in the
    # workspace header starts at whatever the last call (or the fill) left
    shapes = [(700, 512, 4), (270000, 16, 2), (300, 1024, 2), (1300, 512, 8), (270000, 16, 2), (700, 512, 4)]
    size = max(nv.nvfp4_gemv_argmax_workspace_bytes(R, K, n) for R, K, n in shapes)
    wsp = torch.full((size,), 0xFF, dtype=torch.uint8, device=G.DEV)
    for i, (R, K, n) in enumerate(shapes):
        wq, ws, c_ref, s_ref = _prepare(R, K, 100 + R)
        X = G.seeded_x(n, K, seed=200 + i)
        G.note("argmax workspace reuse call %d" % i)
        _, am = G.gemv_argmax_gpu(wq, ws, 1.0, R, K, X, with_logits=False, workspace=wsp)
        Y_ref, _ = oracle.gemv(c_ref, s_ref, 1.0, G.wl.bf16_bits(X))
        assert list(am.cpu().numpy()) == list(oracle.argmax_first(Y_ref)), i


def test_argmax_ties_take_lowest_index():
    R, K = 300, 512
    rng = np.random.default_rng(13)
    codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(0x20, 0x40, (R, K // 16), dtype=np.uint8)
    # plant a row of large positive weights and copy it to later rows
    codes[123] = 0x77
    scales[123] = 0x48
    for r in (5 + 123, 200, 299):
        codes[r], scales[r] = codes[123], scales[123]
    x = torch.ones(2, K, dtype=torch.bfloat16, device=G.DEV)
    cd, sd = G.canonical_to_dev(codes, scales)
    wq, ws = G.repack_gpu(cd, sd, R, K)
    G.note("argmax ties")
    logits, am = G.gemv_argmax_gpu(wq, ws, 1.0, R, K, x)
    assert list(am.cpu().numpy()) == [123, 123]
    Y_ref, _ = oracle.gemv(codes, scales, 1.0, G.wl.bf16_bits(x))
    assert list(oracle.argmax_first(Y_ref)) == [123, 123]
    # all-zero logits: every row ties at 0 (with -0 = +0) -> row 0
    z = torch.zeros(1, K, dtype=torch.bfloat16, device=G.DEV)
    z[0, 0] = -0.0
    _, am0 = G.gemv_argmax_gpu(wq, ws, 1.0, R, K, z)
    assert am0.item() == 0


def test_argmax_ties_across_split_finish_workgroups():
    """Equal maxima in the shares of different finish workgroups (270000
    rows at two columns: 8438 workgroups' keys over the split finish's 16):
    the lowest row wins, as the oracle's first-maximum rule says."""
    R, K = 270000, 16
    rng = np.random.default_rng(17)
    codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(0x20, 0x40, (R, K // 16), dtype=np.uint8)
    codes[269999] = 0x77
    scales[269999] = 0x48
    for r in (140000, 70001, 7):
        codes[r], scales[r] = codes[269999], scales[269999]
    x = torch.ones(2, K, dtype=torch.bfloat16, device=G.DEV)
    cd, sd = G.canonical_to_dev(codes, scales)
    wq, ws = G.repack_gpu(cd, sd, R, K)
    G.note("argmax ties across the split finish")
    _, am = G.gemv_argmax_gpu(wq, ws, 1.0, R, K, x, with_logits=False)
    assert list(am.cpu().numpy()) == [7, 7]
    Y_ref, _ = oracle.gemv(codes, scales, 1.0, G.wl.bf16_bits(x))
    assert list(oracle.argmax_first(Y_ref)) == [7, 7]
    # without row 7 the next one, in another finish workgroup's share
    codes[7] = 0
    cd, sd = G.canonical_to_dev(codes, scales)
    wq, ws = G.repack_gpu(cd, sd, R, K)
    _, am = G.gemv_argmax_gpu(wq, ws, 1.0, R, K, x, with_logits=False)
    assert list(am.cpu().numpy()) == [70001, 70001]


# -------------------------------------------------------------------- SwiGLU

def _check_swiglu(gu: np.ndarray, h_bits: np.ndarray):
    """h must be the nearest-even bf16 of the fp64 SwiGLU; where that value is
    within 1e-6 (relative) of a bf16 rounding midpoint, either neighbour."""
    h64 = oracle.swiglu(gu)
    want = oracle.bf16_rne_array(h64)
    diff = np.nonzero(h_bits != want)[0] if h_bits.ndim == 1 else np.argwhere(h_bits != want)
    for idx in diff:
        idx = tuple(np.atleast_1d(idx))
        v = h64[idx]
        got = float((np.array([h_bits[idx]], np.uint32) << 16).view(np.float32)[0])
        lo_hi = sorted([got, float((np.array([want[idx]], np.uint32) << 16).view(np.float32)[0])])
        mid = 0.5 * (lo_hi[0] + lo_hi[1])
        assert abs(v - mid) <= 1e-6 * abs(v), (idx, v, got)


@pytest.mark.parametrize("F,n", [(17408, 1), (1000, 4), (3, 2)])
def test_swiglu_parity(F, n):
    g = torch.Generator(device=G.DEV).manual_seed(F + n)
    gu = (torch.randn(n, 2 * F, generator=g, device=G.DEV) * 3).to(torch.float32)
    gu[0, 0] = 0.0
    if F > 2:
        gu[0, 1] = 80.0
        gu[0, 2] = -80.0
    h = torch.empty(n, F, dtype=torch.int16, device=G.DEV)
    import block_scaled_bit_nvfp4_amd as nv
    G.note("swiglu F=%d n=%d" % (F, n))
    nv.nvfp4_swiglu(gu, F, n, h)
    _check_swiglu(gu.cpu().numpy(), h.cpu().numpy().view(np.uint16))


# ------------------------------------------- wide product, repeated launches

@pytest.mark.parametrize("R,K,n", [(4160, 2048, 300), (17408, 5120, 512)])
def test_wide_repeat_bit_identical(R, K, n):
    """Forty back-to-back launches of the wide product on the same inputs give
    the same bits as the first, which matches the oracle on sampled rows.  The
    kernel's LDS rings are refilled by direct-to-LDS loads under per-wave
    wait counts and one barrier per octet; a load still in flight at a
    barrier shows up as an occasional differing launch, not as a steady
    error."""
    W = G.seeded_matrix(R, K, 23)
    codes, scales = G.quantize_gpu(W)
    wq, ws = G.repack_gpu(codes, scales, R, K)
    X = G.seeded_x(n, K, seed=24)
    G.note("wide repeat %dx%d n=%d" % (R, K, n))
    first = G.gemv_gpu(wq, ws, 1.0, R, K, X)
    Y = torch.empty_like(first)
    for i in range(40):
        Y.fill_(float("nan"))
        nv.nvfp4_gemv(wq, ws, 1.0, R, K, X, n, Y)
        assert torch.equal(Y.view(torch.int32), first.view(torch.int32)), "launch %d differs" % i
    rows = np.unique(np.concatenate([np.arange(32), np.arange(R - 32, R),
                                     np.random.default_rng(R).choice(R, size=96, replace=False)]))
    c_ref, s_ref = oracle.quantize(W[torch.as_tensor(rows, device=W.device)].cpu().numpy(), 1.0)
    assert np.array_equal(codes[torch.as_tensor(rows, device=W.device)].cpu().numpy(), c_ref)
    Y_ref, S = oracle.gemv(c_ref, s_ref, 1.0, G.wl.bf16_bits(X))
    G.assert_within_tolerance(first.cpu().numpy()[:, rows], Y_ref, S, "wide repeat %dx%d n=%d" % (R, K, n))


@pytest.mark.parametrize("R,K,n", [(8192, 4096, 1), (17408, 5120, 4), (2000, 1024, 8)])
def test_matvec_repeat_bit_identical(R, K, n):
    """Forty back-to-back launches of the matvec, and of its argmax form, give
    the first launch's bits and row indices (the partial sums of a
    workgroup's waves meet in LDS behind one barrier per launch)."""
    W = G.seeded_matrix(R, K, 27)
    codes, scales = G.quantize_gpu(W)
    wq, ws = G.repack_gpu(codes, scales, R, K)
    X = G.seeded_x(n, K, seed=28)
    G.note("matvec repeat %dx%d n=%d" % (R, K, n))
    first = G.gemv_gpu(wq, ws, 1.0, R, K, X)
    logits0, am0 = G.gemv_argmax_gpu(wq, ws, 1.0, R, K, X)
    assert torch.equal(logits0.view(torch.int32), first.view(torch.int32))
    Y = torch.empty_like(first)
    logits = torch.empty_like(first)
    am = torch.empty_like(am0)
    wsp = torch.empty(nv.nvfp4_gemv_argmax_workspace_bytes(R, K, n), dtype=torch.uint8, device=G.DEV)
    for i in range(40):
        Y.fill_(float("nan"))
        nv.nvfp4_gemv(wq, ws, 1.0, R, K, X, n, Y)
        assert torch.equal(Y.view(torch.int32), first.view(torch.int32)), "launch %d differs" % i
        logits.fill_(float("nan"))
        am.fill_(-1)
        nv.nvfp4_gemv_argmax(wq, ws, 1.0, R, K, X, n, logits, am, wsp)
        assert torch.equal(logits.view(torch.int32), first.view(torch.int32)), "argmax launch %d differs" % i
        assert torch.equal(am, am0), "argmax launch %d names other rows" % i
