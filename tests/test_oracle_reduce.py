"""Pins for the reduce arithmetic of the oracle.

The operation (decode, add, re-encode) follows "UCCL-Zip: Lossless
Compression Supercharged GPU Communication", section 3.4 / Figure 6. The
precision: one IEEE binary32 add, then round-half-to-even to BF16. Pins:
  - the BF16 rounding against torch's CPU float32 -> bfloat16 cast (a library
    routine) over every high half and a dense set of low halves;
  - the add against exact rational arithmetic (Python fractions), rounded to
    binary32 and then to BF16 by hand, on random and edge-case pairs;
  - the add against NumPy float64 arithmetic rounded to float32: binary64 has
    at least 2*24+2 significand bits, so rounding the exact sum to binary64
    first and then to binary32 gives the correctly rounded binary32 sum.
The NaN result 0x7FC0 is our convention (parity unpinned by the pages).
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def torch_bf16(u32):
    f = torch.from_numpy(np.ascontiguousarray(u32, dtype=np.uint32).view(np.float32))
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


LOWS = np.array([0x0000, 0x0001, 0x0002, 0x3FFF, 0x7FFE, 0x7FFF, 0x8000, 0x8001,
                 0x8002, 0xBFFF, 0xFFFE, 0xFFFF], dtype=np.uint32)


def test_rne_against_torch_every_high_half():
    hi = np.arange(65536, dtype=np.uint32) << 16
    rng = np.random.default_rng(0)
    lows = np.concatenate([LOWS, rng.integers(0, 65536, 200).astype(np.uint32)])
    for lo in lows:
        u = hi | lo
        f = u.view(np.float32)
        keep = ~np.isnan(f)
        got = oracle.bf16_rne_words(u)
        assert np.array_equal(got[keep], torch_bf16(u[keep])), hex(int(lo))
        assert (got[~keep] == 0x7FC0).all()


@pytest.mark.slow
def test_rne_against_torch_exhaustive():
    step = 1 << 26
    for s in range(0, 1 << 32, step):
        u = np.arange(s, s + step, dtype=np.uint64).astype(np.uint32)
        keep = ~np.isnan(u.view(np.float32))
        got = oracle.bf16_rne_words(u)
        assert np.array_equal(got[keep], torch_bf16(u[keep]))


# ---- exact rational reference ------------------------------------------------
def word_value(w):
    """Exact value of a finite BF16 word as a Fraction (from the IEEE layout)."""
    s = -1 if (w >> 15) & 1 else 1
    E = (w >> 7) & 0xFF
    f = w & 0x7F
    if E == 0:
        return s * Fraction(f, 128) * Fraction(2) ** -126
    return s * (1 + Fraction(f, 128)) * Fraction(2) ** (E - 127)


def round_rational(q: Fraction, p: int, emin: int, emax: int):
    """Round q to a binary format with p significand bits, round half even.
    Returns a Fraction, or +-inf as a float."""
    if q == 0:
        return Fraction(0)
    s = -1 if q < 0 else 1
    a = abs(q)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)                              # subnormal range: fixed quantum
    quantum = Fraction(2) ** (e - (p - 1))
    k = a / quantum
    fl = k.numerator // k.denominator
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** (emax + 1):
        return s * math.inf
    return s * r


def f32_bits_of(v):
    if isinstance(v, float) and math.isinf(v):
        return 0x7F800000 if v > 0 else 0xFF800000
    return int(np.array([float(v)], dtype=np.float64).astype(np.float32).view(np.uint32)[0])


def reference_add(a, b):
    """Exact sum -> binary32 (RNE) -> BF16 (RNE), with IEEE special cases."""
    va, vb = bf16_value_special(a), bf16_value_special(b)
    if isinstance(va, float) or isinstance(vb, float):
        r = float(va) + float(vb)                  # inf / nan cases
        if math.isnan(r):
            return 0x7FC0
        return 0x7F80 if r > 0 else 0xFF80
    q = va + vb
    if q == 0:
        # exact zero sum: -0 only when both are -0 (round to nearest)
        return 0x8000 if (a == 0x8000 and b == 0x8000) else 0x0000
    r32 = round_rational(q, 24, -126, 127)
    if isinstance(r32, float):
        return 0x7F80 if r32 > 0 else 0xFF80
    # r32 is exactly representable in binary32, so this conversion is exact
    u = f32_bits_of(r32)
    r16 = round_rational(r32, 8, -126, 127)
    if isinstance(r16, float):
        return 0x7F80 if r16 > 0 else 0xFF80
    if r16 == 0:
        return 0x8000 if u >> 31 else 0x0000
    return int(np.array([float(r16)], dtype=np.float64).astype(np.float32).view(np.uint32)[0]) >> 16


def bf16_value_special(w):
    E = (w >> 7) & 0xFF
    if E == 0xFF:
        return float("nan") if (w & 0x7F) else (math.inf if not (w >> 15) else -math.inf)
    return word_value(w)


EDGE = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x8080, 0x3F80, 0xBF80,
        0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0, 0x3F81, 0x3B80, 0x4000, 0x0100, 0x7F00]


def test_add_exact_rational_edge_pairs():
    for a in EDGE:
        for b in EDGE:
            assert oracle.add_bf16(a, b) == reference_add(a, b), (hex(a), hex(b))


def test_add_exact_rational_random_pairs():
    rng = np.random.default_rng(42)
    n = 20000
    a = rng.integers(0, 65536, n)
    # bias half the pairs toward close exponents so rounding ties occur
    b = np.where(rng.random(n) < 0.5, rng.integers(0, 65536, n),
                 (a & 0xFF80) ^ rng.integers(0, 0x180, n))
    got = oracle.add_words(a.astype(np.uint16), b.astype(np.uint16))
    for i in range(n):
        assert int(got[i]) == reference_add(int(a[i]), int(b[i])), (hex(a[i]), hex(b[i]))


def test_add_subnormal_sums_are_kept():
    # 2^-133 + 2^-133 = 2^-132: a BF16 subnormal; a flush-to-zero add gives 0
    assert oracle.add_bf16(0x0001, 0x0001) == 0x0002
    # binary32 subnormal sum that BF16 rounds: smallest normal minus a bit
    assert oracle.add_bf16(0x007F, 0x0001) == 0x0080
    assert oracle.add_bf16(0x8001, 0x0001) == 0x0000


def test_add_against_float64_double_rounding_theorem():
    rng = np.random.default_rng(7)
    n = 1 << 21
    a = rng.integers(0, 65536, n).astype(np.uint16)
    b = rng.integers(0, 65536, n).astype(np.uint16)
    fa = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    fb = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    with np.errstate(all="ignore"):
        s32 = (fa + fb).astype(np.float32)
    u = s32.view(np.uint32)
    nan = np.isnan(s32)
    want = np.where(nan, np.uint16(0x7FC0), np.zeros(n, np.uint16))
    want[~nan] = torch_bf16(u[~nan])
    got = oracle.add_words(a, b)
    assert np.array_equal(got, want)


def test_reduce_add_stream_small():
    w = workloads.config(5, small=True)
    A, B = w.x
    cb = oracle.calibrate(A, B)
    sa = oracle.encode(A, 1024, cb.dec)
    sb = oracle.encode(B, 1024, cb.dec)
    r = oracle.reduce_add(sa, sb, A.size, 1024, cb.dec)
    assert oracle.validate(r, cb.dec) == 0
    y = oracle.decode(r, A.size, 1024, cb.dec)
    assert np.array_equal(y, oracle.add_words(A, B))
