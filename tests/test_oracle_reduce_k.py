"""Pins for the oracle's k-input reduce (decode k streams, add each element's
k values in binary32 in input order, round once to BF16, re-encode).

What fixes it other than the oracle itself:
  - k = 2 is the two-input reduce, already pinned against exact rationals and
    torch's binary32 -> BF16 rounding (tests/test_oracle_reduce.py);
  - the summation is checked against NumPy binary32 arithmetic (one IEEE add
    per input, in input order) followed by torch's round-to-nearest-even cast;
  - a hand-derived case where the order of the adds changes the BF16 result;
  - exact rational arithmetic (Python fractions) rounded to binary32 after
    every add, then to BF16, on random tuples;
  - k = 1 re-encodes the input (NaNs become 0x7FC0).
"""
from fractions import Fraction

import numpy as np
import torch

import oracle
import workloads
from test_oracle_reduce import bf16_value_special, round_rational, f32_bits_of


def torch_bf16_of_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def f32_of_words(w):
    return (np.asarray(w, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def numpy_sum(rows):
    """Binary32 sum in row order (NumPy float32 adds are IEEE, round to nearest
    even), then torch's BF16 cast; NaN sums -> 0x7FC0."""
    acc = f32_of_words(rows[0]).copy()
    with np.errstate(all="ignore"):
        for r in rows[1:]:
            acc = (acc + f32_of_words(r)).astype(np.float32)
    out = torch_bf16_of_f32(acc)
    out[np.isnan(acc)] = 0x7FC0
    return out


def test_order_of_the_adds_is_kept():
    # 1 + 2^-8 + 2^-24 + 2^-24, left to right: each 2^-24 lands on a binary32
    # tie (half an ulp of 1 + 2^-8) and rounds back to even, so the sum stays
    # 1 + 2^-8 -- a BF16 tie, which rounds to the even 1.0 (0x3F80).
    # Right to left: 2^-24 + 2^-24 = 2^-23 survives, 1 + 2^-8 + 2^-23 is just
    # above the BF16 tie and rounds up to 1 + 2^-7 (0x3F81). An exact sum
    # rounded once would also give 0x3F81.
    one, e8, e24 = 0x3F80, 0x3B80, 0x3380
    fwd = np.array([[one], [e8], [e24], [e24]], dtype=np.uint16)
    assert oracle.sum_words(fwd)[0] == 0x3F80
    assert oracle.sum_words(fwd[::-1].copy())[0] == 0x3F81


def test_two_inputs_are_the_pairwise_reduce():
    rng = np.random.default_rng(11)
    a = rng.integers(0, 65536, 50000).astype(np.uint16)
    b = rng.integers(0, 65536, 50000).astype(np.uint16)
    assert np.array_equal(oracle.sum_words(np.stack([a, b])), oracle.add_words(a, b))


def test_sum_against_numpy_binary32():
    rng = np.random.default_rng(12)
    for k in (3, 4, 5, 8, 16):
        n = 40000
        # magnitudes within a few binades of each other, so that every add
        # rounds and the order matters; some +-Inf to make Inf - Inf = NaN
        e = rng.integers(110, 140, (k, n))
        m = rng.integers(0, 128, (k, n))
        s = rng.integers(0, 2, (k, n))
        rows = ((s << 15) | (e << 7) | m).astype(np.uint16)
        inf = rng.random((k, n)) < 0.002
        rows[inf] = np.where(rng.random(inf.sum()) < 0.5, 0x7F80, 0xFF80).astype(np.uint16)
        assert np.array_equal(oracle.sum_words(rows), numpy_sum(rows)), k


def reference_sum(words):
    """Exact rational arithmetic: round to binary32 after every add, then BF16."""
    vals = [bf16_value_special(w) for w in words]
    if any(isinstance(v, float) for v in vals):
        return None                                  # specials are covered elsewhere
    acc = vals[0]
    for v in vals[1:]:
        acc = round_rational(acc + v, 24, -126, 127)
        if isinstance(acc, float):
            return None
    r16 = round_rational(acc, 8, -126, 127)
    if isinstance(r16, float):
        return 0x7F80 if r16 > 0 else 0xFF80
    if r16 == 0:
        return None                                  # signed-zero cases: numpy test
    return f32_bits_of(r16) >> 16


def test_sum_against_exact_rationals():
    rng = np.random.default_rng(13)
    checked = 0
    for _ in range(3000):
        k = int(rng.integers(2, 7))
        base = int(rng.integers(100, 150))
        words = [int((rng.integers(0, 2) << 15) | ((base + rng.integers(-6, 7)) << 7) | rng.integers(0, 128))
                 for _ in range(k)]
        want = reference_sum(words)
        if want is None:
            continue
        got = int(oracle.sum_words(np.array(words, dtype=np.uint16).reshape(k, 1))[0])
        assert got == want, [hex(w) for w in words]
        checked += 1
    assert checked > 2500


def test_one_input_reencodes_it():
    rng = np.random.default_rng(14)
    x = rng.integers(0, 65536, 20000).astype(np.uint16)
    cb = oracle.calibrate(x)
    s = oracle.encode(x, 256, cb.dec)
    r = oracle.reduce_k([s], x.size, 256, cb.dec)
    want = x.copy()
    nan = ((x & 0x7F80) == 0x7F80) & ((x & 0x7F) != 0)
    want[nan] = 0x7FC0
    assert np.array_equal(oracle.decode(r, x.size, 256, cb.dec), want)


def test_stream_k_inputs_small():
    w = workloads.config(5, small=True)
    A, B = w.x
    cb = oracle.calibrate(A, B)
    rng = np.random.default_rng(15)
    rows = [A, B] + [(A ^ rng.integers(0, 4, A.size).astype(np.uint16)) for _ in range(3)]
    streams = [oracle.encode(r, 1024, cb.dec) for r in rows]
    r = oracle.reduce_k(streams, A.size, 1024, cb.dec)
    assert oracle.validate(r, cb.dec) == 0
    assert np.array_equal(oracle.decode(r, A.size, 1024, cb.dec), oracle.sum_words(np.stack(rows)))
    # two inputs: the same stream as the pairwise reduce
    assert np.array_equal(oracle.reduce_k(streams[:2], A.size, 1024, cb.dec),
                          oracle.reduce_add(streams[0], streams[1], A.size, 1024, cb.dec))
