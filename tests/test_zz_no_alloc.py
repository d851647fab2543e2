"""uzip_encode_noalloc (the encode that allocates nothing, its workspace a
fixed per-GPU array in the library) against uzip_encode with a caller
workspace: the same stream byte for byte, on two calls in a row whose second
input is smaller, at the largest input the fixed array takes, and the
rejection of a larger one before anything is enqueued."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from lossless_bf16_tensor_amd import uzip

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
C = 1024


def to_dev(x_np):
    return torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).to(DEV)


def largest_n(chunk):
    lo, hi = 1, 1 << 31
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if uzip.workspace_bytes(mid, chunk) <= uzip.NOALLOC_SCRATCH_BYTES:
            lo = mid
        else:
            hi = mid - 1
    return lo


def noalloc_vs_encode(x_np, cb, chunk):
    x = to_dev(x_np)
    n = x_np.size
    cap = uzip.max_bytes(n, chunk)
    ref = torch.full((cap,), 0xEE, dtype=torch.uint8, device=DEV)
    got = torch.full((cap,), 0xEE, dtype=torch.uint8, device=DEV)
    uzip.encode(x, cb, chunk, out=ref)
    uzip.encode_noalloc(x, cb, chunk, out=got)
    torch.cuda.synchronize()
    total, m = uzip.stream_bytes(ref)
    assert uzip.stream_bytes(got) == (total, m)
    assert torch.equal(got[:total], ref[:total]), f"n={n}: streams differ"
    return ref[:total].cpu().numpy(), m


def test_two_calls_second_smaller():
    w = workloads.config(2, small=True)
    ocb = oracle.calibrate(w.calib)
    cb = uzip.codebook_from_hist(ocb.hist)
    rng = np.random.default_rng(7)
    big = w.x
    small = np.ascontiguousarray(rng.permutation(w.x)[:100_003])     # ragged: not a tile or chunk multiple
    s1, m1 = noalloc_vs_encode(big, cb, C)
    s2, m2 = noalloc_vs_encode(small, cb, C)
    assert np.array_equal(s1, oracle.encode(big, C, ocb.dec))
    assert np.array_equal(s2, oracle.encode(small, C, ocb.dec))
    assert m1 > 0 and m2 > 0


def test_largest_input_the_scratch_takes():
    n = largest_n(C)
    rng = np.random.default_rng(11)
    x = rng.integers(0, 1 << 16, n, dtype=np.uint16)             # nearly every exponent an escape
    hist = np.bincount((x[:4096] >> 7) & 0xFF, minlength=256).astype(np.uint64)
    cb = uzip.codebook_from_hist(hist)
    _, m = noalloc_vs_encode(x, cb, C)
    assert m > n // 2
    # one more value needs more workspace than the fixed array holds
    assert uzip.workspace_bytes(n + 1, C) > uzip.NOALLOC_SCRATCH_BYTES
    xb = to_dev(np.zeros(n + 8, dtype=np.uint16))
    out = torch.empty(uzip.max_bytes(n + 8, C), dtype=torch.uint8, device=DEV)
    rc = uzip.lib().uzip_encode_noalloc(uzip._ptr(xb), n + 8, C, uzip.ctypes.byref(cb), uzip._ptr(out), out.numel(),
                                        uzip._stream())
    assert rc == -6 and b"UZIP_NOALLOC_SCRATCH_BYTES" in uzip.lib().uzip_strerror(rc)
