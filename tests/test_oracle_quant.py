"""Pins for the oracle's NVFP4 quantiser: hand-worked blocks, exact-rational
brute force, and invariants of the encoding."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.conftest import golden_lines

E2M1_GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
             Fraction(3), Fraction(4), Fraction(6)]


def _e4m3_finite_magnitudes():
    """All 127 finite non-negative E4M3 values as exact fractions, from the
    bit-field definition enumerated here independently of the oracle."""
    out = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            if e == 0:
                out.append(((e << 3) | m, Fraction(m, 8) * Fraction(1, 64)))
            else:
                out.append(((e << 3) | m, (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)))
    return out


E4M3 = _e4m3_finite_magnitudes()
E4M3_VAL = dict(E4M3)


def _nearest_even(v, table):
    """table: list of (code, value); nearest value to v, ties to even code;
    values beyond the largest saturate."""
    best = None
    for code, val in table:
        d = abs(v - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1]


def quantize_bruteforce(W, tscale):
    """Exact-rational NVFP4 quantisation by exhaustive nearest search."""
    R, K = W.shape
    t = Fraction(float(np.float32(tscale)))
    codes = np.zeros((R, K // 2), np.uint8)
    scales = np.zeros((R, K // 16), np.uint8)
    e2m1_table = list(enumerate(E2M1_GRID))
    for r in range(R):
        for b in range(K // 16):
            blk = [Fraction(float(w)) for w in W[r, 16 * b:16 * b + 16]]
            amax = max(abs(w) for w in blk)
            sb = _nearest_even(amax / (6 * t), E4M3)
            scales[r, b] = sb
            for i in range(16):
                if sb == 0:
                    c = 0
                else:
                    mag = _nearest_even(abs(blk[i]) / (E4M3_VAL[sb] * t), e2m1_table)
                    c = mag | (8 if np.signbit(W[r, 16 * b + i]) else 0)
                k = 16 * b + i
                codes[r, k // 2] |= c << (4 * (k % 2))
    return codes, scales


def test_hand_worked_blocks():
    n = 0
    for line in golden_lines("quantize_blocks.txt"):
        ts, ws, sb, cb = [p.strip() for p in line.split("|")]
        W = np.array([[float(x) for x in ws.split()]], np.float32)
        codes, scales = oracle.quantize(W, float(ts))
        assert scales[0, 0] == int(sb, 16), line
        assert list(codes[0]) == [int(x, 16) for x in cb.split()], (line, [hex(c) for c in codes[0]])
        n += 1
    assert n == 7


@pytest.mark.parametrize("seed,tscale", [(0, 1.0), (1, 0.37), (2, 3.0), (3, 2.0**-7)])
def test_quantize_matches_bruteforce(seed, tscale):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((3, 64)) * 0.02).astype(np.float32)
    W[0, :16] *= 1000.0        # a block whose scale saturates at tscale 1
    W[1, 16:32] = 0.0          # all-zero block
    W[2, 3] = -0.0
    got = oracle.quantize(W, tscale)
    want = quantize_bruteforce(W, tscale)
    assert np.array_equal(got[1], want[1])
    assert np.array_equal(got[0], want[0])


def test_quantize_bruteforce_on_exact_ties():
    # Blocks built from E2M1 tie points times a power-of-two scale, so the
    # element rounding meets exact midpoints everywhere.
    rng = np.random.default_rng(7)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    W = rng.choice(ties, size=(4, 64)) * rng.choice([-1, 1], size=(4, 64))
    W[:, ::16] = 6.0
    W = (W * np.float32(2.0**-5)).astype(np.float32)
    assert np.array_equal(oracle.quantize(W)[0], quantize_bruteforce(W, 1.0)[0])


def _decode_codes(codes):
    lo, hi = codes & 15, codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6] * 2) * np.repeat([1.0, -1.0], 8)
    return grid[c], c


def test_sign_symmetry():
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    c1, s1 = oracle.quantize(W)
    c2, s2 = oracle.quantize(-W)
    assert np.array_equal(s1, s2)
    assert np.array_equal(c1 ^ 0x88, c2)


def test_power_of_two_equivariance():
    rng = np.random.default_rng(12)
    W = (rng.standard_normal((8, 256)) * 0.5).astype(np.float32)
    c0, s0 = oracle.quantize(W)
    s0i = s0.astype(np.int64)
    e0 = (s0i >> 3) & 15
    for j in (-2, -1, 1, 2, 3):
        c1, s1 = oracle.quantize((W * np.float32(2.0**j)).astype(np.float32))
        ok = (e0 >= 1) & (e0 + j >= 1) & (s0i + (j << 3) < 0x7F)
        assert ok.mean() > 0.9
        assert np.array_equal(s1[ok], (s0i[ok] + (j << 3)).astype(np.uint8))
        rows_ok = ok.all(axis=1)
        assert np.array_equal(c1[rows_ok], c0[rows_ok])


def test_error_bound_and_saturation():
    rng = np.random.default_rng(13)
    W = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    W[rng.random(W.shape) < 0.01] = 0.16
    codes, scales = oracle.quantize(W)
    w_hat = oracle.dequant(codes, scales)
    s_blk = np.array([[oracle.e4m3_value(b) for b in row] for row in scales])
    s = np.repeat(s_blk, 16, axis=1)
    _, c = _decode_codes(codes)
    mag = c & 7
    # half the larger grid gap next to each E2M1 magnitude
    half_gap = np.array([0.25, 0.25, 0.25, 0.25, 0.5, 0.5, 1.0, 1.0])
    v = np.abs(W.astype(np.float64)) / s
    err = np.abs(W.astype(np.float64) - w_hat)
    sat = v > 6.0
    assert np.all(err[~sat] <= half_gap[mag[~sat]] * s[~sat])
    assert np.all(err[sat] == np.abs(W[sat].astype(np.float64)) - 6.0 * s[sat])
    # a correctly rounded normal E4M3 scale is within 2^-4 relative of amax/6
    amax = np.abs(W.astype(np.float64)).reshape(16, -1, 16).max(axis=2)
    normal = s_blk >= 2.0**-6
    assert normal.mean() > 0.1      # sigma 0.02 makes most scales subnormal
    assert np.all(amax[normal] / s_blk[normal] <= 6.0 * (1 + 2.0**-4))
    assert np.all(amax[normal] / s_blk[normal] >= 6.0 / (1 + 2.0**-4))
    # subnormal scales have an absolute spacing of 2^-9
    sub = ~normal & (s_blk > 0)
    assert np.all(np.abs(amax[sub] / 6.0 - s_blk[sub]) <= 2.0**-10)


def test_fixed_point_where_a_code_reaches_six():
    rng = np.random.default_rng(14)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    codes, scales = oracle.quantize(W)
    w_hat = oracle.dequant(codes, scales).astype(np.float32)
    codes2, scales2 = oracle.quantize(w_hat)
    _, c = _decode_codes(codes)
    reach6 = ((c & 7) == 7).reshape(8, -1, 16).any(axis=2)
    assert reach6.mean() > 0.3
    assert np.array_equal(scales2[reach6], scales[reach6])
    cb = codes.reshape(8, -1, 8)
    cb2 = codes2.reshape(8, -1, 8)
    assert np.array_equal(cb2[reach6], cb[reach6])
