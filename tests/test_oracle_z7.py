"""Pins for the oracle's Top-7 3-bit + zero-point format (ZipCCL, exponent
coding): round trips over every BF16 word; the printed 16 -> 11 bits
(tests/golden/zipccl_bits.txt); a section by section comparison with the
Top-16 stream of the same input, with the bit planes unpacked by NumPy (the
same sign-mantissa bytes; code k + 1 wherever the Top-16 code k is below 7;
code 0 everywhere else; the zero-point values are those values' exponents in
position order); and the zero-point rate of N(0, 1) samples against the
closed-form mass of the seven most likely exponent octaves."""
import math
import os

import numpy as np
import pytest
from scipy.stats import norm

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
A = lambda v: (v + 255) // 256 * 256


def sec(stream, n, C):
    m = int(np.frombuffer(stream[24:32].tobytes(), np.uint64)[0])
    codes = 256 + A(n)
    P = A((n + 7) // 8)
    offs = codes + 3 * P
    nch = (n + C - 1) // C
    val = offs + A(4 * (nch + 1))
    return m, codes, P, offs, val


def codes_of(stream, n, codes, P):
    planes = [np.unpackbits(stream[codes + b * P:codes + b * P + (n + 7) // 8], bitorder="little")[:n]
              for b in range(3)]
    return planes[0] | (planes[1] << 1) | (planes[2] << 2)


def nibbles(stream, codes, n):
    b = stream[codes:codes + (n + 1) // 2]
    return np.stack([b & 0xF, b >> 4], 1).reshape(-1)[:n]


def test_printed_bit_width():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "zipccl_bits.txt")) if l.strip() and not l.startswith("#")]
    (bits, top, before, after, pct), = [tuple(int(v) for v in r) for r in rows]
    assert top == 2 ** bits - 1                     # one code left for the zero-point
    n = 8 * 4096
    dec = np.array(list(range(120, 136)), np.uint8)
    rng = np.random.default_rng(5)
    e = dec[rng.integers(0, top, n)].astype(np.uint16)
    x = (rng.integers(0, 2, n).astype(np.uint16) << 15) | (e << 7) | rng.integers(0, 128, n).astype(np.uint16)
    cb = oracle.calibrate(np.concatenate([x, (dec[7:].astype(np.uint16) << 7)]))
    assert set(cb.dec[:7]) == set(dec[:7])
    s = oracle.z7_encode(x, 1024, cb.dec)
    assert sec(s, n, 1024)[0] == 0
    assert 8 * oracle.z7_payload_bytes(n, 0) == after * n
    assert before == 16 and round(100 * (1 - after / before)) == pct


@pytest.mark.parametrize("C", [64, 1024, 4096, 65536])
def test_round_trip_every_word(C):
    x = workloads.all_patterns(C + 1)
    cb = oracle.calibrate(x[:5000])
    s = oracle.z7_encode(x, C, cb.dec)
    assert oracle.z7_validate(s, cb.dec) == 0
    assert np.array_equal(oracle.z7_decode(s, x.size, C, cb.dec), x)


@pytest.mark.parametrize("n", [1, 2, 7, 9, 1023, 1025, 50001])
def test_sections_against_top16(n):
    w = workloads.config(1)
    x = w.x[:n].copy()
    cb = oracle.calibrate(w.calib)
    C = 256
    s = oracle.z7_encode(x, C, cb.dec)
    t = oracle.encode(x, C, cb.dec)
    e = (x >> 7) & 0xFF
    in7 = np.isin(e, cb.dec[:7])
    M = int((~in7).sum())
    m, codes, P, offs, val = sec(s, n, C)
    assert m == M
    assert oracle.z7_payload_bytes(n, M) == n + 3 * math.ceil(n / 8) + M
    assert s.size == val + M
    assert np.array_equal(s[256:256 + n], t[256:256 + n])                 # sign-mantissa bytes
    cz = codes_of(s, n, codes, P)
    ct = nibbles(t, 256 + A(n), n)
    assert np.array_equal(cz[in7], ct[in7] + 1)
    assert (cz[~in7] == 0).all()
    assert np.array_equal(s[val:val + M], e[~in7].astype(np.uint8))        # position order
    nch = (n + C - 1) // C
    o = np.frombuffer(s[offs:offs + 4 * (nch + 1)].tobytes(), np.uint32)
    want = np.concatenate([[0], np.cumsum([(~in7[c * C:(c + 1) * C]).sum() for c in range(nch)])])
    assert np.array_equal(o, want)
    # plane bits past n and every padding byte are zero
    for b in range(3):
        tail = np.unpackbits(s[codes + b * P:codes + (b + 1) * P], bitorder="little")[n:]
        assert not tail.any()


def test_zero_point_rate_of_a_gaussian():
    # N(0, 1): the exponent of |x| in [2^k, 2^(k+1)) is 127 + k, with mass
    # 2 (Phi(2^(k+1)) - Phi(2^k)); the seven largest of these masses are the
    # top-7 coverage, and a calibrated codebook's zero-point rate must match
    # one minus it within sampling error.
    ks = np.arange(-40, 10)
    mass = 2 * (norm.cdf(2.0 ** (ks + 1)) - norm.cdf(2.0 ** ks))
    order = np.argsort(-mass, kind="stable")[:7]
    p0 = 1 - mass[order].sum()
    n = 1 << 20
    x = workloads.bf16_bits(np.random.default_rng(9).standard_normal(n))
    cb = oracle.calibrate(x)
    assert sorted(int(v) for v in cb.dec[:7]) == sorted(int(127 + k) for k in ks[order])
    s = oracle.z7_encode(x, 1024, cb.dec)
    m = sec(s, n, 1024)[0]
    assert p0 < 0.03
    assert abs(m / n - p0) < 6 * math.sqrt(p0 * (1 - p0) / n)


def test_special_cases():
    x = workloads.random_words(4096, 3)
    e = (x >> 7) & 0xFF
    vals, cnt = np.unique(e, return_counts=True)
    top = vals[np.argsort(-cnt, kind="stable")][:7]
    xs = x[np.isin(e, top)]
    cb = oracle.calibrate(xs)
    s = oracle.z7_encode(xs, 1024, cb.dec)
    assert sec(s, xs.size, 1024)[0] == 0
    assert np.array_equal(oracle.z7_decode(s, xs.size, 1024, cb.dec), xs)
    # a codebook disjoint from the data: every value is a zero-point
    far = np.array([oracle.merge(0, k) for k in range(200, 216)], dtype=np.uint16)
    lowx = (x & 0x807F) | (np.uint16(10) << 7)
    cbf = oracle.calibrate(far)
    s2 = oracle.z7_encode(lowx, 1024, cbf.dec)
    m, codes, P, offs, val = sec(s2, lowx.size, 1024)
    assert m == lowx.size
    assert not codes_of(s2, lowx.size, codes, P).any()
    assert oracle.z7_payload_bytes(lowx.size, lowx.size) == lowx.size * 2 + 3 * lowx.size // 8
    assert np.array_equal(oracle.z7_decode(s2, lowx.size, 1024, cbf.dec), lowx)


def test_validate_rejects_corruptions():
    w = workloads.config(1)
    x = w.x[:20001].copy()
    cb = oracle.calibrate(w.calib)
    s = oracle.z7_encode(x, 256, cb.dec)
    m, codes, P, offs, val = sec(s, x.size, 256)
    assert m > 0 and oracle.z7_validate(s, cb.dec) == 0
    cz = codes_of(s, x.size, codes, P)
    i = int(np.nonzero(cz == 0)[0][0])
    bad = s.copy(); bad[codes + i // 8] |= 1 << (i % 8)                   # a zero-point becomes code 1
    assert oracle.z7_validate(bad, cb.dec) == -3
    bad = s.copy(); bad[val] = cb.dec[3]                                     # a stored exponent in the top 7
    assert oracle.z7_validate(bad, cb.dec) == -3
    bad = s.copy(); bad[codes + 2 * P + x.size // 8] |= 0x80                 # a plane bit past n
    assert oracle.z7_validate(bad, cb.dec) == -3
    bad = s.copy(); bad[6] = 2
    assert oracle.z7_validate(bad, cb.dec) == -3
    assert oracle.z7_validate(s, np.roll(cb.dec, 1)) == -4
