"""The largest input the library takes: n = 2^32 - 1 values (the chunk
offsets are u32), chunk 1024, a partial last chunk. The words are uniformly
random, so about 15 of every 16 exponents miss the codebook and the escape
count M comes close to 2^32: every 64-bit offset and every 32-bit escape
prefix is exercised near its limit. The oracle cannot encode 8 GiB in
reasonable time, so the test checks what holds at any size (header, M against
a count on the device, bit-exact round trip) and compares sampled chunks with
the oracle's encoding of the same words: the first chunk, the chunks on both
sides of value 2^31, and the partial last chunk."""
import numpy as np
import pytest
import torch

import oracle
from lossless_bf16_tensor_amd import uzip

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
N = (1 << 32) - 1
C = 1024


def A(v):
    return (v + 255) & ~255


def say(msg):
    print(f"[max size] {msg}", flush=True)


def test_maximum_size_round_trip_and_sampled_chunks():
    say(f"n={N} C={C}: generating uniform random words on the device")
    g = torch.Generator(device=DEV)
    g.manual_seed(1234)
    x = torch.randint(-32768, 32768, (N,), dtype=torch.int16, device=DEV, generator=g)
    cal = x[: 1 << 20].cpu().numpy().view(np.uint16)
    ocb = oracle.calibrate(cal)
    cb = uzip.codebook_from_hist(ocb.hist)
    member = torch.zeros(256, dtype=torch.bool, device=DEV)
    member[torch.from_numpy(ocb.dec.astype(np.int64)).to(DEV)] = True

    say("encode")
    out = uzip.encode(x, cb, C)
    total, m = uzip.stream_bytes(out)
    say(f"M={m} total={total}")
    # M against a count of the out-of-codebook exponents on the device
    want_m = 0
    step = 1 << 28
    for i in range(0, N, step):
        e = (x[i:i + step].to(torch.int32) >> 7) & 0xFF
        want_m += int((~member[e.long()]).sum().item())
    assert m == want_m
    assert m < (1 << 32)
    nch = (N + C - 1) // C
    off_codes = 256 + A(N)
    off_offs = off_codes + A((N + 1) // 2)
    off_pos = off_offs + A(4 * (nch + 1))
    off_val = off_pos + A(2 * m)
    assert total == off_val + m

    say("sampled chunks against the oracle")
    for c in (0, (1 << 31) // C - 1, (1 << 31) // C, nch - 1):
        lo = c * C
        ln = min(C, N - lo)
        words = x[lo:lo + ln].cpu().numpy().view(np.uint16)
        sec = oracle.sections(oracle.encode(words, C, ocb.dec))
        sm = out[256 + lo:256 + lo + ln].cpu().numpy()
        codes = out[off_codes + lo // 2:off_codes + lo // 2 + (ln + 1) // 2].cpu().numpy()
        if ln % 2:
            codes = codes.copy()
            codes[-1] &= 0x0F          # the next chunk's first code shares the last byte
        o = out[off_offs + 4 * c:off_offs + 4 * (c + 2)].cpu().numpy().view(np.uint32).astype(np.int64)
        pos = out[off_pos + 2 * o[0]:off_pos + 2 * o[1]].cpu().numpy().view(np.uint16)
        val = out[off_val + o[0]:off_val + o[1]].cpu().numpy()
        assert np.array_equal(sm, sec["sm"]), f"chunk {c}: sign-mantissa bytes"
        assert np.array_equal(codes, sec["codes"]), f"chunk {c}: codes"
        assert np.array_equal(pos, sec["pos"]), f"chunk {c}: positions"
        assert np.array_equal(val, sec["val"]), f"chunk {c}: exponents"

    say("decode")
    y = uzip.decode(out, cb, N, C, in_bytes=total)
    del out
    ok = torch.equal(y, x)
    del x, y
    torch.cuda.empty_cache()
    assert ok
    say("round trip bit-exact")
