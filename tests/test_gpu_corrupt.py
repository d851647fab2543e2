"""Decoding corrupt streams on the GPU. The library bounds every read of a
stream by the caller's byte count, whatever the header, offsets, positions
or codes say: a corrupt stream decodes to wrong values, with no error from
the asynchronous call, no write outside the output and no read outside the
stream, and the structural check reports it. Each corrupted stream sits in a
buffer with 1 MiB of zero slack after it (the byte count passed excludes
it), and the output is a view of a larger buffer whose tail is a canary."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from lossless_bf16_tensor_amd import uzip

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SLACK = 1 << 20
CANARY = 4096


def sections(n, C, fmt):
    A = lambda v: (v + 255) // 256 * 256
    if fmt == "fp8":
        codes = 256 + A((3 * n + 7) // 8)
        offs = codes + A((n + 1) // 2)
    elif fmt == "z7":
        codes = 256 + A(n)
        offs = codes + 3 * A((n + 7) // 8)
    elif fmt == "t8":
        codes = 256 + A(n)
        offs = codes + A((3 * n + 7) // 8)
    else:
        codes = 256 + A(n)
        offs = codes + A((n + 1) // 2)
    pos = offs + A(4 * ((n + C - 1) // C + 1))
    return codes, offs, pos


def corruptions(s, n, C, fmt, rng):
    codes, offs, pos = sections(n, C, fmt)
    out = {}
    b = s.copy(); b[24:32] = np.frombuffer(np.uint64(1 << 40).tobytes(), np.uint8); out["huge M"] = b
    b = s.copy(); b[offs:pos] = rng.integers(0, 256, pos - offs, dtype=np.uint8); out["random offsets"] = b
    b = s.copy(); b[pos:] = rng.integers(0, 256, s.size - pos, dtype=np.uint8); out["random escapes"] = b
    b = s.copy(); b[codes:offs] = rng.integers(0, 256, offs - codes, dtype=np.uint8); out["random codes"] = b
    m = int(np.frombuffer(s[24:32].tobytes(), np.uint64)[0])
    b = s.copy(); b[24:32] = np.frombuffer(np.uint64(m + 1000).tobytes(), np.uint8); out["M too large"] = b
    return out


def on_device(stream_np):
    buf = torch.zeros(stream_np.size + SLACK, dtype=torch.uint8, device=DEV)
    buf[:stream_np.size] = torch.from_numpy(stream_np).to(DEV)
    return buf


def run_case(fmt, n, C, seed):
    rng = np.random.default_rng(seed)
    w = workloads.config(1)
    ocb = oracle.calibrate(w.calib)
    cb = uzip.codebook_from_hist(ocb.hist)
    if fmt == "fp8":
        x = workloads.e5m2_bits(rng.standard_normal(n) * 4.0)
        ocb = oracle.fp8_calibrate(x[: n // 2])
        cb = uzip.codebook_from_hist(ocb.hist)
        s = oracle.fp8_encode(x, C, ocb.dec)
    else:
        x = np.resize(w.x, n).astype(np.uint16)
        s = {"bf16": oracle.encode, "s15": oracle.s15_encode, "z7": oracle.z7_encode,
             "t8": oracle.t8_encode}[fmt](x, C, ocb.dec)
    dec = {"bf16": uzip.decode, "s15": uzip.s15_decode, "z7": uzip.z7_decode, "fp8": uzip.fp8_decode,
           "t8": uzip.t8_decode}[fmt]
    for label, bad in corruptions(s, n, C, fmt, rng).items():
        buf = on_device(bad)
        if fmt == "fp8":
            big = torch.full((n + CANARY,), 0x5A, dtype=torch.uint8, device=DEV)
            canary = 0x5A
        else:
            big = torch.full((n + CANARY,), 0x5A5A, dtype=torch.int16, device=DEV)
            canary = 0x5A5A
        print(f"{fmt} n={n} C={C}: {label}", flush=True)
        dec(buf, cb, n, C, out=big[:n], in_bytes=bad.size)
        torch.cuda.synchronize()
        tail = big[n:].cpu().numpy()
        assert (tail.astype(np.int64) & (0xFF if fmt == "fp8" else 0xFFFF) == canary).all(), f"{label}: write past the output"
        assert uzip.validate(buf, cb, bad.size) != 0, f"{label}: passed the structural check"
    # the device still decodes the intact stream exactly
    y = dec(on_device(s), cb, n, C, in_bytes=s.size).cpu().numpy()
    want = x if fmt == "fp8" else x.view(np.int16)
    assert np.array_equal(y.view(want.dtype), want)


@pytest.mark.parametrize("fmt,n,C", [("bf16", 100003, 1024), ("bf16", 70001, 65536), ("bf16", 50000, 64),
                                     ("s15", 100003, 1024), ("z7", 100003, 1024), ("fp8", 100003, 1024),
                                     ("t8", 100003, 1024), ("t8", 70001, 65536)])
def test_corrupt_stream_decodes_inside_its_buffers(fmt, n, C):
    run_case(fmt, n, C, seed=n + C)


def test_corrupt_input_to_reduce():
    w = workloads.config(1)
    n, C = 100003, 1024
    ocb = oracle.calibrate(w.calib)
    cb = uzip.codebook_from_hist(ocb.hist)
    x = np.resize(w.x, n).astype(np.uint16)
    s = oracle.encode(x, C, ocb.dec)
    rng = np.random.default_rng(9)
    good = on_device(s)
    for label, bad in corruptions(s, n, C, "bf16", rng).items():
        print(f"reduce: {label}", flush=True)
        out = torch.zeros(uzip.max_bytes(n, C) + SLACK, dtype=torch.uint8, device=DEV)
        uzip.reduce_add(good[:s.size], on_device(bad)[:bad.size], cb, n, C, out=out[:uzip.max_bytes(n, C)])
        torch.cuda.synchronize()
        assert not out[uzip.max_bytes(n, C):].any(), f"{label}: write past the output"
