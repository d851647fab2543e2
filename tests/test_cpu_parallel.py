"""The chunk-parallel CPU baseline driver (oracle/parallel.py) is the same
computation as the one-thread oracle: its joined stream equals the oracle's
stream byte for byte, its decode returns the input, and its fused reduce
equals the oracle's, for ragged sizes, every chunk size, all-escape input
and more threads than chunks."""
import numpy as np
import pytest

import oracle
from oracle import parallel


def _input(n, seed, escapes=0.05):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    k = int(escapes * n)
    idx = rng.choice(n, k, replace=False)
    x[idx] = rng.integers(0, 1 << 16, k, dtype=np.uint16)      # any word, many exponents
    return x


@pytest.mark.parametrize("n,chunk,threads", [
    (1, 64, 4), (63, 64, 2), (64, 64, 3), (1000, 64, 7), (4097, 1024, 3),
    (200_003, 1024, 8), (65_536 * 3 + 5, 65_536, 5), (300_000, 4096, 16), (50_000, 256, 1),
])
def test_parallel_stream_equals_oracle(n, chunk, threads):
    x = _input(n, seed=n)
    cb = oracle.calibrate(x[: max(1, n // 4)])
    want = oracle.encode(x, chunk, cb.dec)
    got = parallel.encode_parallel(x, chunk, cb.dec, threads=threads)
    assert got.size == want.size and np.array_equal(got, want)
    y = parallel.decode_parallel(want, n, chunk, cb.dec, threads=threads)
    assert np.array_equal(y, x)


def test_parallel_all_escapes():
    n, chunk = 70_001, 1024
    x = np.full(n, 0x3F80, dtype=np.uint16)                       # exponent 127 only
    cb = oracle.top16(np.bincount([1], minlength=256).astype(np.uint64))   # codebook without 127
    want = oracle.encode(x, chunk, cb.dec)
    assert oracle.stream_m(want) == n
    got = parallel.encode_parallel(x, chunk, cb.dec, threads=6)
    assert np.array_equal(got, want)
    assert np.array_equal(parallel.decode_parallel(want, n, chunk, cb.dec, threads=6), x)


def test_split_then_join_is_identity():
    n, chunk = 123_457, 256
    x = _input(n, seed=9, escapes=0.2)
    cb = oracle.calibrate(x)
    s = oracle.encode(x, chunk, cb.dec)
    bounds = parallel.piece_bounds(n, chunk, 5)
    pieces = [parallel.split(s, *b) for b in bounds]
    for (c0, c1), p in zip(bounds, pieces):
        assert np.array_equal(p, oracle.encode(x[c0 * chunk:min(c1 * chunk, n)], chunk, cb.dec))
    assert np.array_equal(parallel.join(pieces, n, chunk), s)


@pytest.mark.parametrize("n,chunk,threads", [
    (1, 64, 4), (1000, 64, 7), (4097, 1024, 3), (200_003, 1024, 8), (65_536 * 3 + 5, 65_536, 5), (50_000, 256, 1),
])
def test_parallel_reduce_equals_oracle(n, chunk, threads):
    a = _input(n, seed=2 * n + 1)
    b = _input(n, seed=2 * n + 2, escapes=0.2)
    cb = oracle.calibrate(a[: max(1, n // 4)], b[: max(1, n // 4)])
    sa, sb = oracle.encode(a, chunk, cb.dec), oracle.encode(b, chunk, cb.dec)
    want = oracle.reduce_add(sa, sb, n, chunk, cb.dec)
    got = parallel.reduce_add_parallel(sa, sb, n, chunk, cb.dec, threads=threads)
    assert got.size == want.size and np.array_equal(got, want)


@pytest.mark.parametrize("n,threads", [(1, 4), (1000, 7), (200_003, 8), (65_536, 16)])
def test_parallel_histogram_equals_oracle(n, threads):
    x = _input(n, seed=3 * n + 1, escapes=0.3)
    assert np.array_equal(parallel.histogram_parallel(x, threads=threads), oracle.histogram(x))

