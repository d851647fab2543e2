"""Pins for the oracle's Top-8 3-bit format with positions ([SZ] Table 3):
the printed Top-8 ratio from the size formula at the printed escape rate,
round trips over every BF16 word, and a section by section comparison with
the Top-16 stream of the same input, with the 3-bit fields unpacked by NumPy
(the same sign-mantissa bytes; the Top-16 code wherever it is below 8; code 0
and an (in-chunk position, exponent) entry, in position order, for every
other value)."""
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
A = lambda v: (v + 255) // 256 * 256


def sec(stream, n, C):
    m = int(np.frombuffer(stream[24:32].tobytes(), np.uint64)[0])
    codes = 256 + A(n)
    offs = codes + A((3 * n + 7) // 8)
    nch = (n + C - 1) // C
    pos = offs + A(4 * (nch + 1))
    val = pos + A(2 * m)
    return m, codes, offs, pos, val


def codes_of(stream, n, codes):
    bits = np.unpackbits(stream[codes:codes + (3 * n + 7) // 8], bitorder="little")[:3 * n].reshape(n, 3)
    return bits[:, 0] | (bits[:, 1] << 1) | (bits[:, 2] << 2)


def nibbles(stream, codes, n):
    b = stream[codes:codes + (n + 1) // 2]
    return np.stack([b & 0xF, b >> 4], 1).reshape(-1)[:n]


def test_printed_top8_ratio():
    # Table 3's Top-8 row: 7.89 % escapes, ratio 1.241 (no metadata); an
    # input with exactly that escape rate gives it from the oracle's payload
    rows = [l.split() for l in open(os.path.join(GOLDEN, "splitzip_table3.txt")) if l.strip() and not l.startswith("#")]
    bits, cov, esc, ratio, meta = [r for r in rows if r[0] == "3"][0]
    n = 1 << 20
    m = int(round(float(esc) / 100 * n))
    dec = np.arange(100, 116, dtype=np.uint8)
    rng = np.random.default_rng(4)
    e = dec[rng.integers(0, 8, n)].astype(np.uint16)
    idx = rng.choice(n, m, replace=False)
    e[idx] = rng.integers(0, 64, m).astype(np.uint16)          # outside the codebook
    x = (rng.integers(0, 256, n).astype(np.uint16) & 0x807F) | (e << 7)
    cb = oracle.top16(np.r_[np.zeros(100), np.arange(16, 0, -1) * n, np.zeros(140)].astype(np.uint64))
    assert cb.dec.tolist() == dec.tolist()
    s = oracle.t8_encode(x, 1024, cb.dec)
    assert sec(s, n, 1024)[0] == m
    assert 2 * n / oracle.t8_payload_bytes(n, m) == pytest.approx(float(ratio), abs=5e-4)
    assert int(meta) == 0 and 2 * n / s.size < float(ratio)


@pytest.mark.parametrize("C", [64, 1024, 4096, 65536])
def test_round_trip_every_word(C):
    x = workloads.all_patterns(C + 2)
    cb = oracle.calibrate(x[:5000])
    s = oracle.t8_encode(x, C, cb.dec)
    assert oracle.t8_validate(s, cb.dec) == 0
    assert np.array_equal(oracle.t8_decode(s, x.size, C, cb.dec), x)


@pytest.mark.parametrize("n", [1, 2, 7, 9, 1023, 1025, 50001])
def test_sections_against_top16(n):
    w = workloads.config(1)
    x = w.x[:n].copy()
    cb = oracle.calibrate(w.calib)
    C = 256
    s = oracle.t8_encode(x, C, cb.dec)
    t = oracle.encode(x, C, cb.dec)
    e = (x >> 7) & 0xFF
    in8 = np.isin(e, cb.dec[:8])
    M = int((~in8).sum())
    m, codes, offs, pos, val = sec(s, n, C)
    assert m == M
    assert oracle.t8_payload_bytes(n, M) == n + math.ceil(3 * n / 8) + 3 * M
    assert s.size == val + M
    assert np.array_equal(s[256:256 + n], t[256:256 + n])
    c8 = codes_of(s, n, codes)
    c16 = nibbles(t, 256 + A(n), n)
    assert np.array_equal(c8[in8], c16[in8])
    assert (c8[~in8] == 0).all()
    # escapes chunk by chunk in position order
    idx = np.nonzero(~in8)[0]
    assert np.array_equal(np.frombuffer(s[pos:pos + 2 * M].tobytes(), np.uint16), (idx % C).astype(np.uint16))
    assert np.array_equal(s[val:val + M], e[idx].astype(np.uint8))
    nch = (n + C - 1) // C
    o = np.frombuffer(s[offs:offs + 4 * (nch + 1)].tobytes(), np.uint32)
    assert np.array_equal(o, np.searchsorted(idx, np.arange(nch + 1) * C).astype(np.uint32))
    assert not np.unpackbits(s[codes:offs], bitorder="little")[3 * n:].any()


def test_special_cases():
    x = workloads.random_words(4096, 3)
    e = (x >> 7) & 0xFF
    vals, cnt = np.unique(e, return_counts=True)
    top = vals[np.argsort(-cnt, kind="stable")][:8]
    xs = x[np.isin(e, top)]
    cb = oracle.calibrate(xs)
    s = oracle.t8_encode(xs, 1024, cb.dec)
    assert sec(s, xs.size, 1024)[0] == 0
    assert np.array_equal(oracle.t8_decode(s, xs.size, 1024, cb.dec), xs)
    far = np.array([oracle.merge(0, k) for k in range(200, 216)], dtype=np.uint16)
    lowx = (x & 0x807F) | (np.uint16(10) << 7)
    cbf = oracle.calibrate(far)
    s2 = oracle.t8_encode(lowx, 1024, cbf.dec)
    assert sec(s2, lowx.size, 1024)[0] == lowx.size
    assert np.array_equal(oracle.t8_decode(s2, lowx.size, 1024, cbf.dec), lowx)


def test_validate_rejects_corruptions():
    w = workloads.config(1)
    x = w.x[:20001].copy()
    cb = oracle.calibrate(w.calib)
    s = oracle.t8_encode(x, 256, cb.dec)
    m, codes, offs, pos, val = sec(s, x.size, 256)
    assert m > 0 and oracle.t8_validate(s, cb.dec) == 0
    i = 256 * 0 + int(np.frombuffer(s[pos:pos + 2].tobytes(), np.uint16)[0])     # first escape of chunk 0
    bad = s.copy(); bad[codes + (3 * i) // 8] |= 1 << ((3 * i) % 8)            # its code becomes odd
    assert oracle.t8_validate(bad, cb.dec) == -3
    bad = s.copy(); bad[val] = cb.dec[5]                                         # a stored exponent in the codebook
    assert oracle.t8_validate(bad, cb.dec) == -3
    n = x.size
    bad = s.copy(); bad[codes + (3 * n) // 8] |= 0x80                            # a code bit past 3n
    assert oracle.t8_validate(bad, cb.dec) == -3
    bad = s.copy(); bad[6] = 0
    assert oracle.t8_validate(bad, cb.dec) == -3
