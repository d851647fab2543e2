"""Pins for the oracle's calibration sample (the first `sample` words of every
`block` words), checked against a brute-force index predicate."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("n,block,sample", [(1, 8, 8), (7, 8, 8), (100, 16, 8), (1000, 64, 24), (1000, 1000, 8),
                                            (4096, 512, 512), (5000, 4096, 256), (123, 8, 8)])
def test_sample_is_a_prefix_of_every_block(n, block, sample):
    x = np.arange(n, dtype=np.uint16)
    want = np.array([i for i in range(n) if i % block < sample], dtype=np.uint16)
    assert np.array_equal(oracle.sample_words(x, block, sample), want)


def test_block_zero_is_everything():
    x = np.random.default_rng(0).integers(0, 65536, 777).astype(np.uint16)
    assert np.array_equal(oracle.sample_words(x, 0, 0), x)


def test_sampled_codebook_equals_histogram_of_the_sample():
    rng = np.random.default_rng(1)
    x = rng.integers(0, 65536, 20000).astype(np.uint16)
    s = oracle.sample_words(x, 1024, 128)
    assert s.size == sum(min(128, 20000 - b) for b in range(0, 20000, 1024))
    assert np.array_equal(oracle.histogram(s), np.bincount((s >> 7) & 0xFF, minlength=256))
