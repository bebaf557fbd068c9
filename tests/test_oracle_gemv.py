"""Pins for the oracle's dequant, matrix-vector product, SwiGLU, argmax and
repack reference: exact-rational brute force, closed-form special cases,
library routines (scipy's expit) and a hand-derived layout fixture."""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
from tests.conftest import golden_lines

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
        Fraction(3), Fraction(4), Fraction(6)]


def _e2m1_frac(c):
    v = E2M1[c & 7]
    return -v if c & 8 else v


def _e4m3_frac(b):
    e, m = (b >> 3) & 15, b & 7
    v = Fraction(m, 8) / 64 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if b & 0x80 else v


def _bf16_frac(u):
    return Fraction(float(np.array([int(u) << 16], np.uint32).view(np.float32)[0]))


def _random_nvfp4(rng, R, K):
    codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (R, K // 16), dtype=np.uint8)
    scales[(scales & 0x7F) == 0x7F] = 0x7E          # no NaN scales here
    scales[0, 0] = 0x01                               # smallest subnormal
    scales[-1, -1] = 0x7E                             # largest
    return codes, scales


def _random_bf16_bits(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    x *= np.float32(2.0) ** rng.integers(-20, 20, shape).astype(np.float32)
    b = x.view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _w_hat_exact(codes, scales, tscale, r, k):
    byte = int(codes[r, k // 2])
    c = byte & 15 if k % 2 == 0 else byte >> 4
    return _e2m1_frac(c) * _e4m3_frac(int(scales[r, k // 16])) * Fraction(float(np.float32(tscale)))


@pytest.mark.parametrize("R,K,N,tscale", [(4, 32, 1, 1.0), (3, 48, 2, 0.75), (5, 64, 4, 3.0),
                                          (2, 16, 3, 2.0**-20)])
def test_gemv_vs_exact_rationals(R, K, N, tscale):
    rng = np.random.default_rng(R * 100 + K + N)
    codes, scales = _random_nvfp4(rng, R, K)
    X = _random_bf16_bits(rng, (N, K))
    Y, S = oracle.gemv(codes, scales, tscale, X)
    for n in range(N):
        for r in range(R):
            terms = [_w_hat_exact(codes, scales, tscale, r, k) * _bf16_frac(X[n, k]) for k in range(K)]
            exact = sum(terms, Fraction(0))
            mag = sum((abs(t) for t in terms), Fraction(0))
            bound = K * 2.0**-53 * float(mag)
            assert abs(Fraction(Y[n, r]) - exact) <= Fraction(bound), (n, r)
            assert abs(Fraction(S[n, r]) - mag) <= Fraction(bound), (n, r)


def test_every_code_and_scale_reaches_gemv():
    # 16 codes x 256 scales: a 256 x 16 matrix whose row r uses scale byte r
    # and holds every code once; x = 1 on element k picks column k exactly.
    K = 16
    codes = np.tile(np.array([(2 * i) | ((2 * i + 1) << 4) for i in range(8)], np.uint8), (256, 1))
    scales = np.arange(256, dtype=np.uint8)[:, None]
    for k in range(K):
        X = np.zeros((1, K), np.uint16)
        X[0, k] = 0x3F80                                       # 1.0
        Y, _ = oracle.gemv(codes, scales, 1.0, X)
        for r in range(256):
            want = _e2m1_frac(k) * _e4m3_frac(r) if (r & 0x7F) != 0x7F else None
            if want is None:
                assert math.isnan(Y[0, r]) or (k in (0, 8))   # 0 * NaN is NaN; gemv multiplies
            else:
                assert Fraction(Y[0, r]) == want, (k, r)


def test_dequant_vs_exact_rationals():
    rng = np.random.default_rng(5)
    codes, scales = _random_nvfp4(rng, 6, 64)
    for tscale in (1.0, 0.1, 7.5):
        d = oracle.dequant(codes, scales, tscale)
        f32 = oracle.dequant_f32(codes, scales, tscale)
        for r in range(6):
            for k in range(64):
                ex = _w_hat_exact(codes, scales, tscale, r, k)
                assert Fraction(d[r, k]) == ex
                assert f32[r, k] == np.float32(float(ex))   # exact in fp64 -> one rounding


def test_dequant_bf16_is_exact_product():
    rng = np.random.default_rng(6)
    codes, scales = _random_nvfp4(rng, 8, 128)
    bits = oracle.dequant_bf16_bits(codes, scales)
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    for r in range(8):
        for k in range(128):
            assert Fraction(float(vals[r, k])) == _w_hat_exact(codes, scales, 1.0, r, k)


def test_gemv_row_subset_and_special_cases():
    rng = np.random.default_rng(8)
    codes, scales = _random_nvfp4(rng, 40, 96)
    X = _random_bf16_bits(rng, (3, 96))
    Y, S = oracle.gemv(codes, scales, 1.0, X)
    rows = np.array([39, 0, 17, 17])
    Ys, Ss = oracle.gemv_rows(codes, scales, 1.0, X, rows)
    assert np.array_equal(Ys, Y[:, rows]) and np.array_equal(Ss, S[:, rows])
    Yneg, _ = oracle.gemv(codes, scales, 1.0, X ^ np.uint16(0x8000))
    assert np.array_equal(Yneg, -Y)
    Y0, S0 = oracle.gemv(codes, scales, 1.0, np.zeros_like(X))
    assert not Y0.any() and not S0.any()
    Y4, _ = oracle.gemv(codes, scales, 4.0, X)
    assert np.array_equal(Y4, 4.0 * Y)


def test_tolerance_formula():
    S = np.array([0.0, 1.0, 1e5])
    assert np.allclose(oracle.tolerance(S), [1e-6, 1e-5 + 1e-6, 1.0 + 1e-6], rtol=0, atol=1e-15)


def test_argmax_lowest_index_wins_ties():
    Y = np.array([[1.0, 3.0, 3.0, -1.0], [-0.0, 0.0, -5.0, -0.0], [2.0, 1.0, 2.0, 2.0]])
    assert list(oracle.argmax_first(Y)) == [1, 0, 0]
    rng = np.random.default_rng(9)
    Z = rng.standard_normal((4, 1000))
    Z[2, 777] = 100.0
    assert oracle.argmax_first(Z)[2] == 777
    assert list(oracle.argmax_first(Z)) == [int(np.flatnonzero(z == z.max())[0]) for z in Z]


def test_swiglu_vs_scipy_expit():
    rng = np.random.default_rng(10)
    gu = (rng.standard_normal((3, 2 * 500)) * 4).astype(np.float32)
    h = oracle.swiglu(gu)
    g = gu[:, :500].astype(np.float64)
    u = gu[:, 500:].astype(np.float64)
    ref = g * u * scipy.special.expit(g)
    assert np.allclose(h, ref, rtol=4e-16, atol=0)


def test_swiglu_special_values():
    gu = np.array([[0.0, 40.0, -40.0, 1.0, 3.0, 2.0, 5.0, 7.0]], np.float32)
    h = oracle.swiglu(gu)[0]
    assert h[0] == 0.0
    assert h[1] == 40.0 * 2.0                  # exp(-40) is below half an ulp of 1
    assert abs(h[2]) < 1e-15
    assert h[3] == pytest.approx(1.0 * 7.0 / (1.0 + math.e**-1.0), rel=1e-15)
    # silu(g) - silu(-g) = g
    g = np.linspace(-6, 6, 25).astype(np.float32)
    a = oracle.swiglu(np.concatenate([g, np.ones_like(g)])[None])[0]
    b = oracle.swiglu(np.concatenate([-g, np.ones_like(g)])[None])[0]
    assert np.allclose(a - b, g, rtol=0, atol=1e-14)


def test_bf16_rne_array():
    v = np.array([1.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -2.5, 1e-3])
    got = oracle.bf16_rne_array(v)
    assert list(got[:4]) == [0x3F80, 0x3F80, 0x3F82, 0xC020]


def _unrepack(wq, ws, R, K):
    """Inverse of the repacked layout, written from its definition."""
    KB, T = K // 16, (R + 15) // 16
    ST, O = (T + 3) // 4, (KB + 7) // 8
    codes = np.zeros((R, K // 2), np.uint8)
    scales = np.zeros((R, KB), np.uint8)
    cq = wq.reshape(ST, O, 4, 4, 16, 4, 4)    # [st][o][tile][g][r][dword d][byte]
    sq = ws.reshape(ST, O, 4, 16, 8)          # [st][o][tile][r][block in octet]
    for row in range(R):
        st, tt, r = row // 64, (row % 64) // 16, row % 16
        for b in range(KB):
            o, ib = b // 8, b % 8
            for h in range(2):                # element half of the block
                g = 2 * (ib % 2) + h
                codes[row, 8 * b + 4 * h:8 * b + 4 * h + 4] = cq[st, o, tt, g, r, ib // 2]
            scales[row, b] = sq[st, o, tt, r, ib]
    return codes, scales


@pytest.mark.parametrize("R,K", [(17, 32), (16, 1024), (33, 1040), (1, 16), (50, 2064), (130, 272)])
def test_repack_roundtrip_and_padding(R, K):
    rng = np.random.default_rng(R + K)
    codes = rng.integers(1, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(1, 256, (R, K // 16), dtype=np.uint8)
    wq, ws = oracle.repack(codes, scales)
    c2, s2 = _unrepack(wq, ws, R, K)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # a permutation plus zero padding: every nonzero input byte appears once
    assert np.count_nonzero(wq) == codes.size and np.count_nonzero(ws) == scales.size
    assert int(wq.astype(np.int64).sum()) == int(codes.astype(np.int64).sum())


def test_repack_hand_derived_positions():
    R, K = 17, 32
    rng = np.random.default_rng(99)
    codes = rng.integers(1, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(1, 256, (R, K // 16), dtype=np.uint8)
    wq, ws = oracle.repack(codes, scales)
    planes = {"code": wq, "scale": ws}
    n = 0
    for line in golden_lines("repack_17x32.txt"):
        f = line.split()
        if f[0] == "size":
            assert planes[f[1]].size == int(f[2])
            continue
        plane, off = planes[f[0]], int(f[1])
        if f[2] == "zero":
            want = 0
        elif f[2] == "codes":
            want = codes[int(f[3]), int(f[4])]
        else:
            want = scales[int(f[3]), int(f[4])]
        assert plane[off] == want, line
        n += 1
    assert n == 24
