"""Pins for the oracle's FP8 E5M2 variant.

  - the split against the E5M2 value encoding, through torch's float8_e5m2
    type (sign, exponent field, mantissa of every byte), and worked values;
  - the split/merge bijection over all 256 bytes and all (a, e) pairs;
  - the 3-bit packing, read back bit by bit with Python integers;
  - the payload formula ceil(3N/8) + ceil(N/2) + 3M with M counted by NumPy,
    and the page's 1.14x at 0.16 % escapes (tests/golden/splitzip_fp8.txt);
  - exhaustive round trips and the structural checks.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitzip_fp8.txt")


def e5m2_value(b):
    return float(torch.tensor([b], dtype=torch.uint8).view(torch.float8_e5m2).float()[0])


def test_split_against_e5m2_values():
    for b in range(256):
        v = e5m2_value(b)
        e, a = oracle.fp8_exponent(b), oracle.fp8_signmant(b)
        m = a & 3
        if math.isnan(v):
            assert e == 31 and m != 0, b
            continue
        assert (a >> 2) == (1 if math.copysign(1.0, v) < 0 else 0), b
        if math.isinf(v):
            assert e == 31 and m == 0, b
        elif v == 0.0:
            assert e == 0 and m == 0, b
        elif abs(v) < 2.0 ** -14:                      # subnormal: 2^-14 * m / 4
            assert e == 0 and abs(v) == 2.0 ** -14 * m / 4, b
        else:                                          # normal: 2^(e-15) * (1 + m / 4)
            fr, ex = math.frexp(abs(v))
            assert e - 15 == ex - 1, b
            assert abs(v) == 2.0 ** (e - 15) * (1 + m / 4), b


@pytest.mark.parametrize("b,e,a", [(0x3C, 15, 0), (0xBC, 15, 4), (0x7B, 30, 3), (0x7C, 31, 0),
                                   (0x01, 0, 1), (0x80, 0, 4), (0x40, 16, 0), (0x3D, 15, 1)])
def test_worked_values(b, e, a):
    # 0x3C = 1.0, 0xBC = -1.0, 0x7B = 57344 (largest finite), 0x7C = +inf,
    # 0x01 = smallest subnormal, 0x80 = -0, 0x40 = 2.0, 0x3D = 1.25
    assert (oracle.fp8_exponent(b), oracle.fp8_signmant(b)) == (e, a)
    assert oracle.fp8_merge(a, e) == b


def test_bijection():
    for b in range(256):
        assert oracle.fp8_merge(oracle.fp8_signmant(b), oracle.fp8_exponent(b)) == b
    seen = set()
    for a in range(8):
        for e in range(32):
            b = oracle.fp8_merge(a, e)
            assert (oracle.fp8_signmant(b), oracle.fp8_exponent(b)) == (a, e)
            seen.add(b)
    assert len(seen) == 256


def test_histogram_brute_force():
    x = np.random.default_rng(0).integers(0, 256, 5000).astype(np.uint8)
    assert np.array_equal(oracle.fp8_histogram(x), np.bincount((x >> 2) & 31, minlength=256).astype(np.uint64))


def sections(stream, n, C):
    m = int(np.frombuffer(stream[24:32].tobytes(), np.uint64)[0])
    A = lambda v: (v + 255) // 256 * 256
    sm = 256
    codes = sm + A((3 * n + 7) // 8)
    offs = codes + A((n + 1) // 2)
    nch = (n + C - 1) // C
    pos = offs + A(4 * (nch + 1))
    val = pos + A(2 * m)
    return m, sm, codes, offs, pos, val


@pytest.mark.parametrize("n", [1, 7, 8, 9, 15, 16, 17, 100, 1001])
def test_three_bit_packing(n):
    rng = np.random.default_rng(n)
    x = rng.integers(0, 256, n).astype(np.uint8)
    cb = oracle.fp8_calibrate(x)
    s = oracle.fp8_encode(x, 64, cb.dec)
    m, sm, codes, *_ = sections(s, n, 64)
    nbytes = (3 * n + 7) // 8
    big = int.from_bytes(s[sm:sm + nbytes].tobytes(), "little")
    for i in range(n):
        assert (big >> (3 * i)) & 7 == (((int(x[i]) >> 5) & 4) | (int(x[i]) & 3)), i
    assert big >> (3 * n) == 0                       # unused bits are 0
    assert not s[sm + nbytes:codes].any()
    if n == 8:
        assert nbytes == 3


def test_payload_formula_and_worked_ratio():
    rng = np.random.default_rng(5)
    for n in (1000, 4096, 77777):
        x = rng.integers(0, 256, n).astype(np.uint8)
        cb = oracle.fp8_calibrate(x[: n // 2])
        s = oracle.fp8_encode(x, 1024, cb.dec)
        member = np.zeros(256, bool)
        member[cb.dec] = True
        M = int((~member[(x >> 2) & 31]).sum())
        assert sections(s, n, 1024)[0] == M
        assert oracle.fp8_payload_bytes(n, M) == (3 * n + 7) // 8 + (n + 1) // 2 + 3 * M
    # no escape: exactly 8/7 for n a multiple of 8
    assert 8000 / oracle.fp8_payload_bytes(8000, 0) == pytest.approx(8 / 7, abs=0)
    eps, printed, tol = [float(v) for v in open(GOLDEN).read().split("\n")[-2].split()]
    n = 1 << 20
    M = int(round(eps * n))
    assert n / oracle.fp8_payload_bytes(n, M) == pytest.approx(printed, abs=tol)


@pytest.mark.parametrize("C", [64, 256, 1024, 65536])
def test_round_trip_all_bytes(C):
    rng = np.random.default_rng(C)
    x = np.concatenate([rng.permutation(256) for _ in range(40)]).astype(np.uint8)
    for n in (x.size, x.size - 3, 255, 1):
        xs = x[:n]
        cb = oracle.fp8_calibrate(xs)
        s = oracle.fp8_encode(xs, C, cb.dec)
        assert oracle.fp8_validate(s, cb.dec) == 0
        assert np.array_equal(oracle.fp8_decode(s, n, C, cb.dec), xs)


def test_all_escape_and_no_escape():
    x = np.array([oracle.fp8_merge(a, e) for e in range(16, 32) for a in range(8)] * 10, dtype=np.uint8)
    dec = np.arange(16, dtype=np.uint8)               # disjoint from the data: every value escapes
    s = oracle.fp8_encode(x, 256, dec)
    assert sections(s, x.size, 256)[0] == x.size
    assert np.array_equal(oracle.fp8_decode(s, x.size, 256, dec), x)
    dec2 = np.arange(16, 32, dtype=np.uint8)          # covers the data: none escapes
    s2 = oracle.fp8_encode(x, 256, dec2)
    assert sections(s2, x.size, 256)[0] == 0


def test_validate_rejects_corruptions():
    rng = np.random.default_rng(9)
    x = rng.integers(0, 256, 3001).astype(np.uint8)
    cb = oracle.fp8_calibrate(x[:500])
    s = oracle.fp8_encode(x, 256, cb.dec)
    m, sm, codes, offs, pos, val = sections(s, x.size, 256)
    assert m > 0 and oracle.fp8_validate(s, cb.dec) == 0
    bad = s.copy(); bad[6] = 0                      # element type BF16
    assert oracle.fp8_validate(bad, cb.dec) == -3
    bad = s.copy(); bad[sm + (3 * x.size) // 8] |= 0x80   # an unused bit of the last 3-bit byte
    assert oracle.fp8_validate(bad, cb.dec) == -3
    bad = s.copy(); bad[val] = 0x20                 # not a 5-bit exponent
    assert oracle.fp8_validate(bad, cb.dec) == -3
    bad = s.copy(); bad[val] = cb.dec[0]            # an escape inside the codebook
    assert oracle.fp8_validate(bad, cb.dec) == -3
    assert oracle.fp8_validate(s, np.roll(cb.dec, 1)) == -4
