"""GPU parity of online calibration: the sampled histogram, and encodes whose
codebook is calibrated on the device from the input itself. Every stream
must equal the oracle's encode under the oracle's own calibration of the
same sample, and the device-written codebook must equal the oracle's."""
import ctypes

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


def host_words(t):
    return t.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n,block,sample", [(1, 8, 8), (1000, 64, 24), (100003, 4096, 512), (100003, 8, 8),
                                            (1 << 20, 1 << 16, 1 << 13), (77777, 80000, 8)])
def test_sampled_histogram(n, block, sample):
    x = workloads.random_words(n, 3) & np.uint16(0x8FFF)          # a skewed exponent mix
    h = uzip.histogram(to_dev(x), block=block, sample=sample).cpu().numpy().astype(np.uint64)
    assert np.array_equal(h, oracle.histogram(oracle.sample_words(x, block, sample)))


def check_online(x_np, C, block, sample, label):
    dev_cb = torch.zeros(ctypes.sizeof(uzip.Codebook), dtype=torch.uint8, device=DEV)
    buf = uzip.encode_online(to_dev(x_np), C, block, sample, cb_out=dev_cb)
    total, m = uzip.stream_bytes(buf)
    ocb = oracle.calibrate(oracle.sample_words(x_np, block, sample))
    want = oracle.encode(x_np, C, ocb.dec)
    got = buf[:total].cpu().numpy()
    assert total == want.size, f"{label}: size {total} != {want.size}"
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        pytest.fail(f"{label}: {bad.size} bytes differ, first at {bad[:8].tolist()}")
    cb = uzip.codebook_of_device(dev_cb)
    assert list(cb.dec) == ocb.dec.tolist()
    assert np.array_equal(np.array(cb.enc), ocb.enc) and np.array_equal(np.array(cb.member), ocb.member)
    assert np.array_equal(np.array(cb.hist, dtype=np.uint64), ocb.hist)
    assert cb.n_cal == int(ocb.hist.sum()) and cb.version == uzip.UZIP_VERSION
    # a receiver rebuilds the codebook from the header alone
    hdr = uzip.parse_header(buf[:256].cpu().numpy().tobytes())
    rcb = uzip.codebook_from_dec(hdr["dec"])
    y = host_words(uzip.decode(buf, rcb, x_np.size, C, in_bytes=total))
    assert np.array_equal(y, x_np), label
    return buf, total, m


def test_online_config1():
    w = workloads.config(1)
    check_online(w.x, 1024, 0, 0, "config 1 online")


@pytest.mark.parametrize("C", [64, 1024, 65536])
def test_online_config3_small(C):
    w = workloads.config(3, small=True)
    check_online(w.x, C, 0, 0, f"config 3 small online C={C}")
    check_online(w.x, C, 1 << 14, 1 << 11, f"config 3 small sampled C={C}")


@pytest.mark.parametrize("n", [1, 9, 8191, 8193, 100003])
def test_online_ragged(n):
    x = workloads.random_words(n, 8)
    check_online(x, 1024, 0, 0, f"random n={n}")
    check_online(x, 256, 64, 16, f"random n={n} sampled")


def test_online_all_patterns():
    check_online(workloads.all_patterns(2), 4096, 0, 0, "all words")


def test_online_pooled_calls_do_not_leak():
    # two calls in a row on the same workspace: the second codebook must come
    # from the second input only
    ws = torch.empty(uzip.workspace_bytes(50000, 1024), dtype=torch.uint8, device=DEV)
    a = workloads.random_words(50000, 1)
    b = (workloads.random_words(50000, 2) & np.uint16(0x83FF)) | np.uint16(0x3C00)
    for x in (a, b):
        buf = uzip.encode_online(to_dev(x), 1024, ws=ws)
        total, _ = uzip.stream_bytes(buf)
        want = oracle.encode(x, 1024, oracle.calibrate(x).dec)
        assert np.array_equal(buf[:total].cpu().numpy(), want)


@pytest.mark.timeout(900)
def test_online_config3_full():
    w = workloads.config(3)
    print("config 3: input ready", flush=True)
    check_online(w.x, 1024, 0, 0, "config 3 online (whole input)")
    print("config 3: whole-input calibration ok", flush=True)
    check_online(w.x, 1024, 1 << 20, 1 << 17, "config 3 online (256 KiB of every 2 MiB)")
