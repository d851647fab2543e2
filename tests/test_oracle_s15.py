"""Pins for the oracle's Top-15 + sentinel format: round trips over every
BF16 word, the payload N + N/2 + M with M counted by NumPy, and a section by
section comparison with the Top-16 stream of the same input (the same
sign-mantissa bytes; the same codes wherever the exponent is one of the 15;
code 15 everywhere else; the stored exponents are those values' exponents
in position order)."""
import numpy as np
import pytest

import oracle
import workloads


def sec(stream, n, C, s15):
    m = int(np.frombuffer(stream[24:32].tobytes(), np.uint64)[0])
    A = lambda v: (v + 255) // 256 * 256
    codes = 256 + A(n)
    offs = codes + A((n + 1) // 2)
    nch = (n + C - 1) // C
    pos = offs + A(4 * (nch + 1))
    val = pos if s15 else pos + A(2 * m)
    return m, codes, offs, pos, val


def nibbles(stream, codes, n):
    b = stream[codes:codes + (n + 1) // 2]
    return np.stack([b & 0xF, b >> 4], 1).reshape(-1)[:n]


@pytest.mark.parametrize("C", [64, 256, 1024, 4096, 65536])
def test_round_trip_every_word(C):
    x = workloads.all_patterns(C)
    cb = oracle.calibrate(x[:5000])
    s = oracle.s15_encode(x, C, cb.dec)
    assert oracle.s15_validate(s, cb.dec) == 0
    assert np.array_equal(oracle.s15_decode(s, x.size, C, cb.dec), x)


@pytest.mark.parametrize("n", [1, 2, 7, 1023, 1025, 50001])
def test_sections_against_top16(n):
    w = workloads.config(1)
    x = w.x[:n].copy()
    cb = oracle.calibrate(w.calib)
    C = 256
    s = oracle.s15_encode(x, C, cb.dec)
    t = oracle.encode(x, C, cb.dec)
    e = (x >> 7) & 0xFF
    in15 = np.isin(e, cb.dec[:15])
    M = int((~in15).sum())
    m, codes, offs, pos, val = sec(s, n, C, True)
    assert m == M
    assert oracle.s15_payload_bytes(n, M) == n + (n + 1) // 2 + M
    assert s.size == val + M
    assert np.array_equal(s[256:256 + n], t[256:256 + n])                 # sign-mantissa bytes
    cs = nibbles(s, codes, n)
    ct = nibbles(t, sec(t, n, C, False)[1], n)
    assert np.array_equal(cs[in15], ct[in15])
    assert (cs[~in15] == 15).all()
    assert np.array_equal(s[val:val + M], e[~in15].astype(np.uint8))       # position order
    # chunk offsets count the sentinels chunk by chunk
    nch = (n + C - 1) // C
    o = np.frombuffer(s[offs:offs + 4 * (nch + 1)].tobytes(), np.uint32)
    want = np.concatenate([[0], np.cumsum([(~in15[c * C:(c + 1) * C]).sum() for c in range(nch)])])
    assert np.array_equal(o, want)


def test_special_cases():
    x = workloads.random_words(4096, 3)
    dec = np.unique((x >> 7) & 0xFF)
    # a codebook whose first 15 entries cover every exponent: no escapes, 4/3
    e = (x >> 7) & 0xFF
    vals, cnt = np.unique(e, return_counts=True)
    top = vals[np.argsort(-cnt, kind="stable")][:15]
    xs = x[np.isin(e, top)]
    cb = oracle.calibrate(xs)
    s = oracle.s15_encode(xs, 1024, cb.dec)
    assert sec(s, xs.size, 1024, True)[0] == 0
    # a codebook disjoint from the data: every value escapes, 2.5 N payload
    far = np.array([oracle.merge(0, k) for k in range(200, 216)], dtype=np.uint16)
    lowx = (x & 0x807F) | (np.uint16(10) << 7)
    cbf = oracle.calibrate(far)
    s2 = oracle.s15_encode(lowx, 1024, cbf.dec)
    assert sec(s2, lowx.size, 1024, True)[0] == lowx.size
    assert oracle.s15_payload_bytes(lowx.size, lowx.size) == int(2.5 * lowx.size)
    assert np.array_equal(oracle.s15_decode(s2, lowx.size, 1024, cbf.dec), lowx)


def test_validate_rejects_corruptions():
    w = workloads.config(1)
    x = w.x[:20000].copy()
    cb = oracle.calibrate(w.calib)
    s = oracle.s15_encode(x, 256, cb.dec)
    m, codes, offs, pos, val = sec(s, x.size, 256, True)
    assert m > 0 and oracle.s15_validate(s, cb.dec) == 0
    cs = nibbles(s, codes, x.size)
    i = int(np.nonzero(cs == 15)[0][0])
    bad = s.copy(); bad[codes + i // 2] &= (0xF0 if i % 2 == 0 else 0x0F)    # a sentinel becomes code 0
    assert oracle.s15_validate(bad, cb.dec) == -3
    bad = s.copy(); bad[val] = cb.dec[3]                                       # a stored exponent in the book
    assert oracle.s15_validate(bad, cb.dec) == -3
    bad = s.copy(); bad[6] = 0
    assert oracle.s15_validate(bad, cb.dec) == -3
