"""Pins for the oracle's element and scale codes (decode and round-to-nearest-even encode).

Each check compares the oracle against something other than itself: a value
table from the format specifications (tests/golden/), torch's float8_e4m3fn
and bfloat16 conversions (library routines), or exact-rational brute force.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import golden_lines


def test_e2m1_table_matches_spec_listing():
    seen = 0
    for line in golden_lines("e2m1_values.txt"):
        code, val = line.split()
        got = oracle.e2m1_value(int(code))
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)
        seen += 1
    assert seen == 16


def test_e2m1_via_torch_e4m3_decode():
    # An E2M1 code with exponent e >= 1 and mantissa m equals the E4M3 byte
    # with exponent e + 6 and mantissa m << 2 (both have value 2^(e-1)(1+m/2));
    # the E2M1 subnormal 0.5 is the E4M3 normal 2^-1 (byte 0x30).
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        if e == 0 and m == 0:
            byte = 0
        elif e == 0:
            byte = 0x30
        else:
            byte = ((e + 6) << 3) | (m << 2)
        byte |= s << 7
        ref = torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item()
        assert oracle.e2m1_value(code) == ref, code


def test_e4m3_all_256_codes_vs_torch():
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double()
    for b in range(256):
        got = oracle.e4m3_value(b)
        ref = t[b].item()
        if math.isnan(ref):
            assert math.isnan(got), b
        else:
            assert got == ref and math.copysign(1, got) == math.copysign(1, ref), (b, got, ref)
    assert sum(math.isnan(oracle.e4m3_value(b)) for b in range(256)) == 2


def test_e4m3_landmarks_from_spec():
    for line in golden_lines("e4m3_special.txt"):
        b, v = line.split()
        got = oracle.e4m3_value(int(b, 16))
        if v == "nan":
            assert math.isnan(got)
        else:
            assert got == float(v) and math.copysign(1, got) == math.copysign(1, float(v)), b


def test_e4m3_encode_roundtrip_all_finite():
    for b in range(0x7F):
        assert oracle.e4m3_encode(oracle.e4m3_value(b)) == b


def test_e4m3_encode_vs_torch_cast_random_and_midpoints():
    rng = np.random.default_rng(1)
    # log-uniform over the whole finite range, plus every midpoint (exact ties)
    vals = list(np.exp(rng.uniform(np.log(2.0**-12), np.log(448.0), 4000)).astype(np.float32))
    for b in range(0x7E):
        lo, hi = oracle.e4m3_value(b), oracle.e4m3_value(b + 1)
        vals.append(np.float32((lo + hi) / 2))
        vals.append(np.nextafter(np.float32((lo + hi) / 2), np.float32(0)))
        vals.append(np.nextafter(np.float32((lo + hi) / 2), np.float32(1e9)))
    vals = np.array(vals, np.float32)
    vals = vals[vals <= 448.0]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in vals], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), int(got[i]), int(ref[i])) for i in bad[:5]]


def test_e4m3_encode_saturates_and_underflows():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(463.999) == 0x7E
    assert oracle.e4m3_encode(464.0) == 0x7E      # would be 480 (a NaN code): saturate
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(2.0**-10) == 0x00   # tie between 0 and 2^-9 -> even (0)
    assert oracle.e4m3_encode(2.0**-10 * 1.0000001) == 0x01
    assert oracle.e4m3_encode(0.0) == 0x00


def test_e2m1_encode_ties_table():
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for line in golden_lines("e2m1_ties.txt"):
        v, want = map(float, line.split())
        assert grid[oracle.e2m1_encode_mag(v)] == want, v


def _e2m1_bruteforce(v: Fraction) -> int:
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
            Fraction(3), Fraction(4), Fraction(6)]
    best = None
    for c, g in enumerate(grid):
        d = abs(v - g)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_e2m1_encode_bruteforce_random():
    rng = np.random.default_rng(2)
    vals = list(rng.uniform(0, 8, 3000)) + [k / 8 for k in range(0, 64)]
    for v in vals:
        assert oracle.e2m1_encode_mag(float(v)) == _e2m1_bruteforce(Fraction(float(v))), v


def test_bf16_rne_vs_torch_cast():
    rng = np.random.default_rng(3)
    f = rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32)
    f = f[np.isfinite(f)]
    # exact ties: a bf16 value plus half its ulp (representable in fp32)
    base = torch.from_numpy(f).to(torch.bfloat16).float().numpy()
    ties = (base.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    vals = np.concatenate([f, ties[np.isfinite(ties)], np.array([0.0, -0.0, 1e-40, -3e-39], np.float32)])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_rne(float(v)) for v in vals], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_bf16_value_decodes_bits():
    for bits, want in [(0x3F80, 1.0), (0xBF80, -1.0), (0x4040, 3.0), (0x0001, 2.0**-133),
                       (0x7F7F, float(np.float32(3.3895313892515355e38)))]:
        assert oracle.bf16_value(bits) == want
