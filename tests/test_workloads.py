"""The seeded input generators: fixed draws, the stated shapes, the BF16 and
E5M2 casts (torch's round to nearest even), and the structure each recipe
promises."""
import numpy as np
import pytest

import workloads


def test_casts_round_to_nearest_even():
    # 1 + 2^-8 is halfway between BF16 1.0 and 1 + 2^-7: ties to even (1.0);
    # 1 + 3 * 2^-8 ties up to 1 + 2^-6
    v = workloads.bf16_bits([1.0, -2.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 0.0, float("inf")])
    assert v.tolist() == [0x3F80, 0xC000, 0x3F80, 0x3F82, 0x0000, 0x7F80]
    e = workloads.e5m2_bits([1.0, -2.0, 0.5, 57344.0])
    assert e.tolist() == [0x3C, 0xC0, 0x38, 0x7B]


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_configs_are_deterministic_and_shaped(k):
    a = workloads.config(k, small=True)
    b = workloads.config(k, small=True)
    xa = a.x if isinstance(a.x, tuple) else (a.x,)
    xb = b.x if isinstance(b.x, tuple) else (b.x,)
    for u, v in zip(xa, xb):
        assert u.dtype == np.uint16 and np.array_equal(u, v)
        assert u.size == int(np.prod(a.shape))
    assert a.name == workloads.CONFIG_NAMES[k]


def test_kv_cache_layer_scales():
    # per-layer scales are log-uniform over [0.05, 20]: the median |x| of
    # the layers spreads over several octaves, K and V of a layer alike
    w = workloads.config_3(tokens=16, layers=8)
    f = w.x.astype(np.uint32) << 16
    x = f.view(np.float32).reshape(2, 8, 16 * 8 * 128)
    med = np.median(np.abs(x), axis=2)
    assert np.log2(med.max() / med.min()) > 3
    assert np.all(np.abs(np.log2(med[0] / med[1])) < 3)


def test_reduce_shards_and_e5m2_cache():
    w = workloads.reduce_shards(k=3, buckets=2, bucket=1 << 12)
    assert len(w.x) == 3 and all(s.size == 2 << 12 for s in w.x)
    assert not np.array_equal(w.x[0], w.x[1])
    e = workloads.kv_cache_e5m2(tokens=8, layers=2)
    assert e.x.dtype == np.uint8 and e.x.size == 2 * 2 * 8 * 8 * 128


def test_all_patterns_is_a_permutation():
    p = workloads.all_patterns(3)
    assert np.array_equal(np.sort(p), np.arange(65536, dtype=np.uint16))
