"""Pins for the oracle's split / merge / histogram / Top-16.

The split is checked against IEEE-754 semantics (frexp on the decoded value),
not against its own bit formula, so a wrong shift or mask fails here.
Source of the operations: "SplitZip: Ultra Fast Lossless KV Compression for
Disaggregated LLM Serving", section 3.2 (split/merge), section 3.3
(histogram, Top-16, three tables).
"""
import collections
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_value(word: int) -> float:
    return float(np.array([word << 16], dtype=np.uint32).view(np.float32)[0])


def ieee_fields(word: int):
    """(biased exponent, sign-mantissa byte) of a BF16 word from its value.

    BF16 keeps binary32's 8-bit exponent and the top 7 fraction bits, so a
    finite value is (-1)^s * 2^(E-127) * (1 + f/128) for E >= 1 and
    (-1)^s * 2^-126 * f/128 for E = 0. NaN has no value to decompose and
    returns None."""
    v = bf16_value(word)
    if math.isnan(v):
        return None
    s = 1 if math.copysign(1.0, v) < 0 else 0
    av = abs(v)
    if av == 0.0:
        E, f = 0, 0
    elif math.isinf(av):
        E, f = 255, 0
    else:
        m, k = math.frexp(av)          # av = m * 2^k, 0.5 <= m < 1
        if k - 1 >= -126:
            E = k - 1 + 127
            frac = (2.0 * m - 1.0) * 128.0
        else:
            E = 0
            frac = av / 2.0 ** -133
        f = int(frac)
        assert f == frac and 0 <= f < 128
    return E, (s << 7) | f


def test_worked_value_from_page():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "split_worked_values.txt"))
            if l.strip() and not l.startswith("#")]
    assert rows
    for w, e, a in rows:
        w, e, a = int(w, 16), int(e), int(a, 16)
        assert oracle.exponent(w) == e
        assert oracle.signmant(w) == a
        assert oracle.merge(a, e) == w


@pytest.mark.parametrize("word,e,a", [
    (0x3F80, 127, 0x00), (0xBF80, 127, 0x80), (0x8000, 0, 0x80), (0x0000, 0, 0x00),
    (0x7F80, 255, 0x00), (0xFF80, 255, 0x80), (0x0001, 0, 0x01), (0xC000, 128, 0x80),
    (0x7F7F, 254, 0x7F), (0x0080, 1, 0x00),
])
def test_special_words(word, e, a):
    # the expected fields come from the value, not from the bit formula
    if not math.isnan(bf16_value(word)):
        assert ieee_fields(word) == (e, a)
    assert (oracle.exponent(word), oracle.signmant(word)) == (e, a)


def test_split_matches_ieee_semantics_all_words():
    nan_count = 0
    for w in range(65536):
        f = ieee_fields(w)
        e, a = oracle.exponent(w), oracle.signmant(w)
        if f is None:
            nan_count += 1
            assert e == 255 and (a & 0x7F) != 0          # NaN: all-ones exponent, nonzero fraction
            assert (a >> 7) == (w >> 15)                  # sign bit kept
        else:
            assert (e, a) == f, hex(w)
    assert nan_count == 2 * 127


def test_merge_inverts_split_all_words():
    for w in range(65536):
        assert oracle.merge(oracle.signmant(w), oracle.exponent(w)) == w


def test_split_of_merge_is_identity_all_pairs():
    seen = set()
    for e in range(256):
        for a in range(256):
            w = oracle.merge(a, e)
            assert oracle.exponent(w) == e and oracle.signmant(w) == a
            seen.add(w)
    assert len(seen) == 65536        # (a, e) <-> word is a bijection


@pytest.mark.parametrize("seed,n", [(0, 1), (1, 7), (2, 1000), (3, 4097)])
def test_histogram_brute_force(seed, n):
    x = workloads.random_words(n, seed)
    want = collections.Counter()
    for w in x.tolist():
        f = ieee_fields(w)
        want[255 if f is None else f[0]] += 1
    h = oracle.histogram(x)
    assert int(h.sum()) == n
    for e in range(256):
        assert int(h[e]) == want.get(e, 0)


def test_histogram_constant_and_pooled():
    x = np.full(12345, 0x3F80, dtype=np.uint16)
    h = oracle.histogram(x)
    assert int(h[127]) == 12345 and int(h.sum()) == 12345
    a = workloads.random_words(5000, 7)
    b = workloads.random_words(3000, 8)
    assert np.array_equal(oracle.histogram(a, b), oracle.histogram(a) + oracle.histogram(b))


def _check_tables(cb):
    assert len(set(cb.dec.tolist())) == 16
    for k in range(16):
        assert cb.enc[cb.dec[k]] == k
    assert set(np.nonzero(cb.member)[0].tolist()) == set(cb.dec.tolist())
    for e in range(256):
        if not cb.member[e]:
            assert cb.enc[e] == 0


def test_top16_equal_counts_take_smallest_exponents():
    h = np.zeros(256, dtype=np.uint64)
    h[200:220] = 9
    cb = oracle.top16(h)
    assert cb.dec.tolist() == list(range(200, 216))
    _check_tables(cb)


def test_top16_fewer_than_16_distinct():
    h = np.zeros(256, dtype=np.uint64)
    h[130], h[7], h[250] = 5, 100, 5
    cb = oracle.top16(h)
    fill = [e for e in range(256) if e not in (7, 130, 250)][:13]
    assert cb.dec.tolist() == [7, 130, 250] + fill
    _check_tables(cb)


@pytest.mark.parametrize("seed", range(6))
def test_top16_brute_force_and_dominance(seed):
    rng = np.random.default_rng(seed)
    h = rng.integers(0, 40, 256).astype(np.uint64)      # many ties
    cb = oracle.top16(h)
    want = sorted(range(256), key=lambda e: (-int(h[e]), e))[:16]
    assert cb.dec.tolist() == want
    sel = [int(h[e]) for e in cb.dec]
    rest = [int(h[e]) for e in range(256) if not cb.member[e]]
    assert min(sel) >= max(rest)
    assert sel == sorted(sel, reverse=True)
    _check_tables(cb)


def test_calibration_on_config1():
    w = workloads.config_1()
    cb = oracle.calibrate(w.calib)
    # N(0,1): the most frequent exponents sit just below 127 (|x| in [0.5, 1))
    assert cb.dec[0] in (126, 127)
    assert int(cb.hist.sum()) == w.calib.size
