"""GPU parity of the FP8 E5M2 variant against the oracle: histograms,
codebooks, byte-identical streams and exact round trips."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from lossless_bf16_tensor_amd import uzip

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def to_dev(x_np):
    return torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.uint8)).to(DEV)


def check(x_np, C, cb, ocb, label):
    buf = uzip.fp8_encode(to_dev(x_np), cb, C)
    total, m = uzip.stream_bytes(buf)
    want = oracle.fp8_encode(x_np, C, ocb.dec)
    got = buf[:total].cpu().numpy()
    assert total == want.size, f"{label}: size {total} != {want.size}"
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        pytest.fail(f"{label}: {bad.size} bytes differ, first at {bad[:8].tolist()}")
    y = uzip.fp8_decode(buf, cb, x_np.size, C, in_bytes=total).cpu().numpy()
    if not np.array_equal(y, x_np):
        bad = np.nonzero(y != x_np)[0]
        pytest.fail(f"{label} decode: {bad.size} values differ, first {bad[:8].tolist()}")
    return buf, total, m


def codebooks(x_np):
    ocb = oracle.fp8_calibrate(x_np)
    return uzip.codebook_from_hist(ocb.hist), ocb


def test_histogram_and_calibrate():
    x = workloads.kv_cache_e5m2(tokens=8, layers=8).x
    h = uzip.fp8_histogram(to_dev(x)).cpu().numpy().astype(np.uint64)
    assert np.array_equal(h, oracle.fp8_histogram(x))
    cb = uzip.fp8_calibrate(to_dev(x))
    assert list(cb.dec) == oracle.fp8_calibrate(x).dec.tolist()
    for n in (1, 15, 17, 100003):
        xs = workloads.random_words(n, n).astype(np.uint8)
        assert np.array_equal(uzip.fp8_histogram(to_dev(xs)).cpu().numpy().astype(np.uint64),
                              oracle.fp8_histogram(xs))


@pytest.mark.parametrize("C", [64, 256, 1024, 4096, 65536])
def test_all_bytes_every_chunk(C):
    rng = np.random.default_rng(C)
    x = np.concatenate([rng.permutation(256) for _ in range(300)]).astype(np.uint8)
    cb, ocb = codebooks(x)
    check(x, C, cb, ocb, f"all bytes C={C}")


# 680 and 8872 put the end of the 3-bit section 1 byte short of a 256-byte
# boundary with a partial last group of values
@pytest.mark.parametrize("n", [1, 7, 8, 9, 31, 32, 33, 680, 4095, 4096, 4097, 8191, 8192, 8193, 8872, 100003])
def test_ragged_sizes(n):
    x = workloads.random_words(n, 1000 + n).astype(np.uint8)
    cb, ocb = codebooks(x[: max(1, n // 2)])
    check(x, 1024, cb, ocb, f"n={n}")


def test_all_escape_and_no_escape():
    x = np.array([oracle.fp8_merge(a, e) for e in range(16, 32) for a in range(8)] * 300, dtype=np.uint8)
    ocb = oracle.fp8_calibrate(np.array([oracle.fp8_merge(0, e) for e in range(16)], dtype=np.uint8))
    cb = uzip.codebook_from_hist(ocb.hist)
    _, _, m = check(x, 256, cb, ocb, "all escapes")
    assert m == x.size
    cb2, ocb2 = codebooks(x)
    _, _, m2 = check(x, 256, cb2, ocb2, "no escapes")
    assert m2 == 0


def test_kv_cache_small():
    w = workloads.kv_cache_e5m2(tokens=8, layers=8)
    cb, ocb = codebooks(w.calib)
    for C in (64, 1024, 65536):
        check(w.x, C, cb, ocb, f"e5m2 kv small C={C}")


def test_deterministic():
    x = workloads.random_words(300001, 4).astype(np.uint8)
    cb, _ = codebooks(x)
    a = uzip.fp8_encode(to_dev(x), cb, 1024)
    b = uzip.fp8_encode(to_dev(x), cb, 1024)
    ta, _ = uzip.stream_bytes(a)
    assert torch.equal(a[:ta], b[:ta])


@pytest.mark.timeout(900)
def test_kv_cache_full():
    w = workloads.kv_cache_e5m2()
    print(f"{w.name}: input ready", flush=True)
    cb = uzip.fp8_calibrate(to_dev(w.calib))
    ocb = oracle.fp8_calibrate(w.calib)
    assert list(cb.dec) == ocb.dec.tolist()
    check(w.x, 1024, cb, ocb, "e5m2 kv cache 2^28")


def test_worked_example_stream():
    # the FP8 stream worked out by hand (tests/golden/stream_fp8_worked_example.txt)
    from test_oracle_format import BYTES_FP8, CHUNK, GOLDEN_FP8, golden_stream
    calib = np.repeat(np.array([0x3C, 0x40, 0x00], dtype=np.uint8), [10, 5, 3])
    cb = uzip.codebook_from_hist(oracle.fp8_calibrate(calib).hist)
    want = golden_stream(GOLDEN_FP8)
    buf = uzip.fp8_encode(torch.from_numpy(BYTES_FP8).to(DEV), cb, CHUNK)
    total, m = uzip.stream_bytes(buf)
    assert (total, m) == (want.size, 1)
    assert np.array_equal(buf[:total].cpu().numpy(), want)
    y = uzip.fp8_decode(buf, cb, BYTES_FP8.size, CHUNK, in_bytes=total).cpu().numpy()
    assert np.array_equal(y, BYTES_FP8)
