"""GPU parity of the Top-8 3-bit format with positions against the oracle: identical
streams and exact round trips."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from lossless_bf16_tensor_amd import uzip

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def to_dev(x_np):
    return torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).to(DEV)


def check(x_np, C, cb, ocb, label):
    buf = uzip.t8_encode(to_dev(x_np), cb, C)
    total, m = uzip.stream_bytes(buf)
    want = oracle.t8_encode(x_np, C, ocb.dec)
    got = buf[:total].cpu().numpy()
    assert total == want.size, f"{label}: size {total} != {want.size}"
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        pytest.fail(f"{label}: {bad.size} bytes differ, first at {bad[:8].tolist()}")
    y = uzip.t8_decode(buf, cb, x_np.size, C, in_bytes=total).cpu().numpy().view(np.uint16)
    if not np.array_equal(y, x_np):
        bad = np.nonzero(y != x_np)[0]
        pytest.fail(f"{label} decode: {bad.size} words differ, first {bad[:8].tolist()}")
    return buf, total, m


def codebooks(calib):
    ocb = oracle.calibrate(calib)
    return uzip.codebook_from_hist(ocb.hist), ocb


@pytest.mark.parametrize("C", [64, 256, 1024, 4096, 65536])
def test_all_words(C):
    x = workloads.all_patterns(C)
    cb, ocb = codebooks(x[:3000])
    check(x, C, cb, ocb, f"all words C={C}")


@pytest.mark.parametrize("n", [1, 2, 7, 8, 9, 1023, 4095, 4096, 4097, 8191, 8192, 8193, 100003])
def test_ragged(n):
    w = workloads.config(1)
    x = np.resize(w.x, n).astype(np.uint16)
    cb, ocb = codebooks(w.calib)
    check(x, 1024, cb, ocb, f"n={n}")


def test_dense_escapes():
    # every word an escape: exponents 0..15 only, codebook from far exponents
    x = (workloads.random_words(70001, 5) & np.uint16(0x87FF)).astype(np.uint16)
    far = np.array([oracle.merge(0, k) for k in range(200, 216)], dtype=np.uint16)
    cb, ocb = codebooks(far)
    _, _, m = check(x, 256, cb, ocb, "all escapes")
    assert m == x.size


def test_configs_small():
    for k in (1, 2, 4):
        w = workloads.config(k, small=True)
        cb, ocb = codebooks(w.calib)
        for C in (256, 1024, 4096):
            check(w.x, C, cb, ocb, f"config {k} small C={C}")


@pytest.mark.timeout(900)
def test_config3_full():
    w = workloads.config(3)
    print(f"{w.name}: input ready", flush=True)
    cb, ocb = codebooks(w.calib)
    check(w.x, 1024, cb, ocb, "config 3 Top-8 3-bit")


def test_eight_codes_no_escapes():
    # exponents only from the top 8: no escapes, 11 bits per value
    rng = np.random.default_rng(8)
    dec = np.arange(120, 136, dtype=np.uint16)
    n = 50000
    e = dec[rng.integers(0, 8, n)]
    x = ((rng.integers(0, 2, n).astype(np.uint16) << 15) | (e << 7) | rng.integers(0, 128, n).astype(np.uint16))
    cb, ocb = codebooks(np.concatenate([x, dec[8:] << 7]).astype(np.uint16))
    _, total, m = check(x.astype(np.uint16), 1024, cb, ocb, "no escapes")
    assert m == 0


def test_chunks_larger_than_the_decode_tile():
    w = workloads.config(4, small=True)
    cb, ocb = codebooks(w.calib)
    for C in (8192, 65536):
        check(w.x, C, cb, ocb, f"config 4 small C={C}")


def test_device_validate_and_reuse():
    # a GPU stream passes the structural check; a second, smaller encode into
    # the same buffers gives the oracle's stream again
    w = workloads.config(2, small=True)
    cb, ocb = codebooks(w.calib)
    n = w.x.size
    out = torch.empty(uzip.t8_max_bytes(n, 1024), dtype=torch.uint8, device=DEV)
    ws = torch.empty(uzip.workspace_bytes(n, 1024), dtype=torch.uint8, device=DEV)
    for k in (n, n // 3 + 5):
        x = w.x[:k].copy()
        uzip.t8_encode(to_dev(x), cb, 1024, out=out, ws=ws)
        total, _ = uzip.stream_bytes(out)
        assert uzip.validate(out, cb, total) == 0
        assert np.array_equal(out[:total].cpu().numpy(), oracle.t8_encode(x, 1024, ocb.dec))
