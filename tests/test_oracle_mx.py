"""Pins of the oracle's MXFP4 part (the second block-scaled format: E2M1
codes, one E8M0 power-of-two scale per 32 elements) against what does not
come from the oracle: torch's float8_e8m0fnu decoding, hand-worked blocks
(tests/golden/mx_quantize_blocks.txt, derived from the OCP Microscaling
MXFP4 definition), an exact-rational brute force, invariants, exact dot
products, and hand-derived byte positions of the repacked layout."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1_MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
             Fraction(6)]


def test_e8m0_all_bytes_match_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for i in range(256):
        v = oracle.e8m0_value(i)
        if np.isnan(ref[i]):
            assert np.isnan(v) and i == 255
        else:
            assert v == ref[i], i


def _parse_weight(tok):
    return float.fromhex(tok) if "0x" in tok.lower() else float(tok)


def _golden_blocks():
    out = []
    for line in open(os.path.join(GOLDEN, "mx_quantize_blocks.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        ts, ws, sb, cb = [p.strip() for p in line.split("|")]
        w = [_parse_weight(t) for t in ws.split()]
        w += [0.0] * (32 - len(w))
        out.append((float(ts), np.array(w, np.float32), int(sb, 16), bytes.fromhex(cb)))
    return out


@pytest.mark.parametrize("case", range(8))
def test_quantize_hand_worked_blocks(case):
    ts, w, sbyte, cbytes = _golden_blocks()[case]
    codes, scales = oracle.mx_quantize(w[None, :], ts)
    assert int(scales[0, 0]) == sbyte
    assert bytes(codes[0]) == cbytes


def _brute_block(w, tscale):
    """Exact-rational MXFP4 of one block: the E with 4 <= amax/(tscale 2^E) < 8
    (clamped to [-127, 127]), then per element the nearest E2M1 magnitude by
    exhaustive search, ties to the even code, saturating at 6."""
    q = max(abs(Fraction(float(x))) for x in w) / Fraction(float(tscale))
    if q == 0:
        E = -127
    else:
        E = 0
        while q >= Fraction(8) * Fraction(2) ** E:
            E += 1
        while q < Fraction(4) * Fraction(2) ** E:
            E -= 1
        E = min(max(E, -127), 127)
    denom = Fraction(2) ** E * Fraction(float(tscale))
    codes = []
    for x in w:
        v = abs(Fraction(float(x))) / denom
        best = None
        for c, m in enumerate(E2M1_MAGS):
            d = abs(v - m)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        codes.append(best[1] | (8 if np.signbit(x) else 0))
    return E + 127, codes


@pytest.mark.parametrize("seed", range(6))
def test_quantize_brute_force(seed):
    rng = np.random.default_rng(seed)
    blocks = []
    for i in range(40):
        mag = 2.0 ** rng.integers(-20, 20)
        w = (rng.standard_normal(32) * mag).astype(np.float32)
        if i % 5 == 0:   # exact E2M1 ties at a power-of-two scale
            e = int(rng.integers(-8, 8))
            w = (rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], 32) * 2.0 ** e
                 * rng.choice([-1, 1], 32)).astype(np.float32)
        blocks.append(w)
    W = np.stack(blocks)
    for ts in (1.0, 0.375):
        codes, scales = oracle.mx_quantize(W, ts)
        for r, w in enumerate(W):
            sb, cs = _brute_block(w, ts)
            assert int(scales[r, 0]) == sb
            got = [(int(codes[r, i // 2]) >> (4 * (i % 2))) & 15 for i in range(32)]
            assert got == cs, (seed, r)


def test_quantize_power_of_two_equivariance():
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    c0, s0 = oracle.mx_quantize(W)
    for j in (-9, 3, 20):
        c1, s1 = oracle.mx_quantize((W * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1.astype(int), s0.astype(int) + j)


def test_dequant_exact_and_gemv_exact_on_tiny_shapes():
    rng = np.random.default_rng(3)
    R, K = 5, 64
    codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(100, 150, (R, K // 32), dtype=np.uint8)
    for ts in (1.0, 0.75):
        wh = oracle.mx_dequant(codes, scales, ts)
        X = rng.standard_normal((2, K)).astype(np.float32)
        xb = (torch.from_numpy(X).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
        Y, S = oracle.mx_gemv(codes, scales, ts, xb)
        for r in range(R):
            exact_w = []
            for k in range(K):
                c = (int(codes[r, k // 2]) >> (4 * (k % 2))) & 15
                m = E2M1_MAGS[c & 7] * (-1 if c & 8 else 1)
                w = m * Fraction(2) ** (int(scales[r, k // 32]) - 127) * Fraction(ts)
                assert Fraction(float(wh[r, k])) == w
                exact_w.append(w)
            for n in range(2):
                x = [Fraction(float(torch.tensor(int(b)).to(torch.int16).view(torch.bfloat16).item()))
                     for b in xb[n].astype(np.int16)]
                exact = sum(a * b for a, b in zip(exact_w, x))
                mag = sum(abs(a * b) for a, b in zip(exact_w, x))
                assert abs(Fraction(Y[n, r]) - exact) <= mag * Fraction(K, 2 ** 52)
                assert abs(Fraction(S[n, r]) - mag) <= mag * Fraction(K, 2 ** 52)


def test_repack_byte_positions():
    # R = 17 rows (one row into the second tile), K = 160: five 32-element
    # blocks, two octets of 128 elements (the second partial).
    R, K = 17, 160
    codes = (np.arange(R * K // 2) % 251 + 1).astype(np.uint8).reshape(R, K // 2)
    scales = (np.arange(R * K // 32) % 200 + 3).astype(np.uint8).reshape(R, K // 32)
    wq, ws = oracle.mx_repack(codes, scales)
    O = 2
    assert wq.size == 1 * O * 4 * 64 * 16 and ws.size == 1 * O * 4 * 16 * 4

    def code_entry(o, tt, l):
        return wq[((o * 4 + tt) * 64 + l) * 16:((o * 4 + tt) * 64 + l) * 16 + 16]

    # row 0, lane g = 0 of octet 0: dword d = code bytes 16 d .. 16 d + 3
    assert bytes(code_entry(0, 0, 0)) == bytes(np.concatenate([codes[0, 16 * d:16 * d + 4] for d in range(4)]))
    # row 5, lane group 3 (l = 53): bytes 16 d + 12 .. +15
    assert bytes(code_entry(0, 0, 53)[8:12]) == bytes(codes[5, 44:48])
    # row 16 is tile 1, r = 0; octet 1 holds block 4 (code bytes 64..79), d = 0
    assert bytes(code_entry(1, 1, 32)[0:4]) == bytes(codes[16, 72:76])
    # octet 1 past the row's end (d = 1..3) and rows past 17 are zero
    assert not code_entry(1, 1, 32)[4:].any()
    assert not code_entry(0, 1, 1).any()
    # scale plane [ST][O][4][16][4]: byte i of (o, tt, r) is block 4o + i
    assert ws[((0 * 4 + 0) * 16 + 3) * 4 + 2] == scales[3, 2]
    assert ws[((1 * 4 + 0) * 16 + 7) * 4 + 0] == scales[7, 4]
    assert ws[((1 * 4 + 1) * 16 + 0) * 4 + 0] == scales[16, 4]
    assert ws[((1 * 4 + 1) * 16 + 0) * 4 + 1] == 0
    # the code plane is the NVFP4 code plane of the same codes
    wq_nv, _ = oracle.repack(codes, np.zeros((R, K // 16), np.uint8))
    assert np.array_equal(wq, wq_nv)
