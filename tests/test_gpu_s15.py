"""GPU parity of the Top-15 + sentinel format against the oracle: identical
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
    buf = uzip.s15_encode(to_dev(x_np), cb, C)
    total, m = uzip.stream_bytes(buf)
    want = oracle.s15_encode(x_np, C, ocb.dec)
    got = buf[:total].cpu().numpy()
    assert total == want.size, f"{label}: size {total} != {want.size}"
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        pytest.fail(f"{label}: {bad.size} bytes differ, first at {bad[:8].tolist()}")
    y = uzip.s15_decode(buf, cb, x_np.size, C, in_bytes=total).cpu().numpy().view(np.uint16)
    if not np.array_equal(y, x_np):
        bad = np.nonzero(y != x_np)[0]
        pytest.fail(f"{label} decode: {bad.size} words differ, first {bad[:8].tolist()}")
    return buf, total, m


def codebooks(calib):
    ocb = oracle.calibrate(calib)
    return uzip.codebook_from_hist(ocb.hist), ocb


@pytest.mark.parametrize("C", [64, 256, 1024, 4096])
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
    check(w.x, 1024, cb, ocb, "config 3 Top-15 + sentinel")
