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


def test_maximum_size_fp8():
    """The same at n = 2^32 - 1 E5M2 bytes. The codebook is calibrated on
    bytes whose exponent is below 16 (bit 6 of the byte clear), so it holds
    exponents 0..15; the data are uniform bytes with bit 6 also set in about
    a fifth of them, so about 60 % of the exponents (16..31) are escapes and
    M is well above 2^31."""
    say(f"E5M2 n={N} C={C}: generating random bytes on the device")
    g = torch.Generator(device=DEV)
    g.manual_seed(4321)
    x = torch.randint(0, 256, (N,), dtype=torch.uint8, device=DEV, generator=g)
    step = 1 << 28
    for i in range(0, N, step):
        r = torch.randint(0, 256, (min(step, N - i),), dtype=torch.uint8, device=DEV, generator=g)
        x[i:i + step] |= (r < 51).to(torch.uint8) << 6
    cal = x[: 1 << 20].cpu().numpy() & 0xBF
    ocb = oracle.fp8_calibrate(cal)
    assert sorted(ocb.dec.tolist()) == list(range(16))
    cb = uzip.codebook_from_hist(ocb.hist)
    member = torch.zeros(32, dtype=torch.bool, device=DEV)
    member[torch.from_numpy(ocb.dec.astype(np.int64)).to(DEV)] = True

    say("encode")
    out = uzip.fp8_encode(x, cb, C)
    total, m = uzip.stream_bytes(out)
    say(f"M={m} total={total}")
    want_m = 0
    for i in range(0, N, step):
        e = (x[i:i + step].to(torch.int32) >> 2) & 0x1F
        want_m += int((~member[e.long()]).sum().item())
    assert m == want_m
    assert (1 << 31) < m < (1 << 32)
    nch = (N + C - 1) // C
    sm_bytes = (3 * N + 7) // 8
    off_codes = 256 + A(sm_bytes)
    off_offs = off_codes + A((N + 1) // 2)
    off_pos = off_offs + A(4 * (nch + 1))
    off_val = off_pos + A(2 * m)
    assert total == off_val + m

    say("sampled chunks against the oracle")
    for c in (0, (1 << 31) // C - 1, (1 << 31) // C, nch - 1):
        lo = c * C
        ln = min(C, N - lo)
        mini = oracle.fp8_encode(x[lo:lo + ln].cpu().numpy(), C, ocb.dec)
        mm = int(mini[24:32].view(np.uint64)[0])
        msm = (3 * ln + 7) // 8
        mcodes = 256 + A(msm)
        mpos = mcodes + A((ln + 1) // 2) + A(8)          # one chunk: two offsets
        mval = mpos + A(2 * mm)
        sm = out[256 + 3 * lo // 8:256 + 3 * lo // 8 + msm].cpu().numpy()
        codes = out[off_codes + lo // 2:off_codes + lo // 2 + (ln + 1) // 2].cpu().numpy()
        o = out[off_offs + 4 * c:off_offs + 4 * (c + 2)].cpu().numpy().view(np.uint32).astype(np.int64)
        pos = out[off_pos + 2 * o[0]:off_pos + 2 * o[1]].cpu().numpy().view(np.uint16)
        val = out[off_val + o[0]:off_val + o[1]].cpu().numpy()
        assert np.array_equal(sm, mini[256:256 + msm]), f"chunk {c}: sign-mantissa bits"
        assert np.array_equal(codes, mini[mcodes:mcodes + (ln + 1) // 2]), f"chunk {c}: codes"
        assert np.array_equal(pos, mini[mpos:mpos + 2 * mm].view(np.uint16)), f"chunk {c}: positions"
        assert np.array_equal(val, mini[mval:mval + mm]), f"chunk {c}: exponents"

    say("decode")
    y = uzip.fp8_decode(out, cb, N, C, in_bytes=total)
    del out
    ok = torch.equal(y, x)
    del x, y
    torch.cuda.empty_cache()
    assert ok
    say("round trip bit-exact")


def test_maximum_size_reduce():
    """The fused reduce at n = 2^32 - 1: two inputs of uniformly random words
    (so the sum's escapes also number more than 2^31). Checked: the output's
    M against a count over its decoded words, sampled chunks of the output
    stream against the oracle's reduce of the same chunks of the inputs, and
    2^20 sampled sums against the oracle's add."""
    say(f"reduce n={N} C={C}: generating two inputs on the device")
    g = torch.Generator(device=DEV)
    g.manual_seed(99)
    a = torch.randint(-32768, 32768, (N,), dtype=torch.int16, device=DEV, generator=g)
    b = torch.randint(-32768, 32768, (N,), dtype=torch.int16, device=DEV, generator=g)
    ocb = oracle.calibrate(a[: 1 << 20].cpu().numpy().view(np.uint16), b[: 1 << 20].cpu().numpy().view(np.uint16))
    cb = uzip.codebook_from_hist(ocb.hist)
    member = torch.zeros(256, dtype=torch.bool, device=DEV)
    member[torch.from_numpy(ocb.dec.astype(np.int64)).to(DEV)] = True

    say("encode both, reduce")
    sa = uzip.encode(a, cb, C)
    ta = uzip.stream_bytes(sa)[0]
    sb = uzip.encode(b, cb, C)
    tb = uzip.stream_bytes(sb)[0]
    out = uzip.reduce_add(sa[:ta], sb[:tb], cb, N, C)
    del sa, sb
    total, m = uzip.stream_bytes(out)
    say(f"M={m} total={total}")
    nch = (N + C - 1) // C
    off_codes = 256 + A(N)
    off_offs = off_codes + A((N + 1) // 2)
    off_pos = off_offs + A(4 * (nch + 1))
    off_val = off_pos + A(2 * m)
    assert total == off_val + m
    assert (1 << 31) < m < (1 << 32)

    say("sampled chunks against the oracle's reduce")
    for c in (0, (1 << 31) // C - 1, (1 << 31) // C, nch - 1):
        lo = c * C
        ln = min(C, N - lo)
        wa = a[lo:lo + ln].cpu().numpy().view(np.uint16)
        wb = b[lo:lo + ln].cpu().numpy().view(np.uint16)
        mini = oracle.reduce_add(oracle.encode(wa, C, ocb.dec), oracle.encode(wb, C, ocb.dec), ln, C, ocb.dec)
        sec = oracle.sections(mini)
        sm = out[256 + lo:256 + lo + ln].cpu().numpy()
        codes = out[off_codes + lo // 2:off_codes + lo // 2 + (ln + 1) // 2].cpu().numpy()
        o = out[off_offs + 4 * c:off_offs + 4 * (c + 2)].cpu().numpy().view(np.uint32).astype(np.int64)
        pos = out[off_pos + 2 * o[0]:off_pos + 2 * o[1]].cpu().numpy().view(np.uint16)
        val = out[off_val + o[0]:off_val + o[1]].cpu().numpy()
        assert np.array_equal(sm, sec["sm"]), f"chunk {c}: sign-mantissa bytes"
        assert np.array_equal(codes, sec["codes"]), f"chunk {c}: codes"
        assert np.array_equal(pos, sec["pos"]), f"chunk {c}: positions"
        assert np.array_equal(val, sec["val"]), f"chunk {c}: exponents"

    say("decode, M over the decoded sums, sampled sums against the oracle")
    y = uzip.decode(out, cb, N, C, in_bytes=total)
    del out
    want_m = 0
    step = 1 << 28
    for i in range(0, N, step):
        e = (y[i:i + step].to(torch.int32) >> 7) & 0xFF
        want_m += int((~member[e.long()]).sum().item())
    assert m == want_m
    idx = torch.randint(0, N, (1 << 20,), device=DEV, generator=g)
    got = y[idx].cpu().numpy().view(np.uint16)
    want = oracle.add_words(a[idx].cpu().numpy().view(np.uint16), b[idx].cpu().numpy().view(np.uint16))
    del a, b, y
    torch.cuda.empty_cache()
    assert np.array_equal(got, want)
    say("reduce checked")


def test_maximum_size_reduce_k():
    """The k-input reduce at n = 2^32 - 1 with three inputs of uniformly
    random words (the sum's escapes number more than 2^31). Checked: the
    output's M against a count over its decoded words, sampled chunks of the
    output stream against the oracle's reduce of the same chunks of the
    inputs, and 2^20 sampled sums against the oracle's in-order sums."""
    k = 3
    say(f"reduce_k k={k} n={N} C={C}: generating the inputs on the device")
    g = torch.Generator(device=DEV)
    g.manual_seed(123)
    xs = [torch.randint(-32768, 32768, (N,), dtype=torch.int16, device=DEV, generator=g) for _ in range(k)]
    ocb = oracle.calibrate(*[x[: 1 << 20].cpu().numpy().view(np.uint16) for x in xs])
    cb = uzip.codebook_from_hist(ocb.hist)
    member = torch.zeros(256, dtype=torch.bool, device=DEV)
    member[torch.from_numpy(ocb.dec.astype(np.int64)).to(DEV)] = True
    nch = (N + C - 1) // C
    chunks = (0, (1 << 31) // C - 1, (1 << 31) // C, nch - 1)
    # the words the checks need, kept on the host before the inputs are freed
    words = {c: [x[c * C:c * C + min(C, N - c * C)].cpu().numpy().view(np.uint16) for x in xs] for c in chunks}
    idx = torch.randint(0, N, (1 << 20,), device=DEV, generator=g)
    rows = np.stack([x[idx].cpu().numpy().view(np.uint16) for x in xs])

    say("encode the inputs, reduce")
    streams = []
    for i in range(k):
        si = uzip.encode(xs[i], cb, C)
        streams.append(si[:uzip.stream_bytes(si)[0]])
        xs[i] = None
    del xs
    torch.cuda.empty_cache()
    out = uzip.reduce_k(streams, cb, N, C)
    del streams
    torch.cuda.empty_cache()
    total, m = uzip.stream_bytes(out)
    say(f"M={m} total={total}")
    off_codes = 256 + A(N)
    off_offs = off_codes + A((N + 1) // 2)
    off_pos = off_offs + A(4 * (nch + 1))
    off_val = off_pos + A(2 * m)
    assert total == off_val + m
    assert (1 << 31) < m < (1 << 32)

    say("sampled chunks against the oracle's reduce")
    for c in chunks:
        lo = c * C
        ln = min(C, N - lo)
        mini = oracle.reduce_k([oracle.encode(w, C, ocb.dec) for w in words[c]], ln, C, ocb.dec)
        sec = oracle.sections(mini)
        sm = out[256 + lo:256 + lo + ln].cpu().numpy()
        codes = out[off_codes + lo // 2:off_codes + lo // 2 + (ln + 1) // 2].cpu().numpy()
        o = out[off_offs + 4 * c:off_offs + 4 * (c + 2)].cpu().numpy().view(np.uint32).astype(np.int64)
        pos = out[off_pos + 2 * o[0]:off_pos + 2 * o[1]].cpu().numpy().view(np.uint16)
        val = out[off_val + o[0]:off_val + o[1]].cpu().numpy()
        assert np.array_equal(sm, sec["sm"]), f"chunk {c}: sign-mantissa bytes"
        assert np.array_equal(codes, sec["codes"]), f"chunk {c}: codes"
        assert np.array_equal(pos, sec["pos"]), f"chunk {c}: positions"
        assert np.array_equal(val, sec["val"]), f"chunk {c}: exponents"

    say("decode, M over the decoded sums, sampled sums against the oracle")
    y = uzip.decode(out, cb, N, C, in_bytes=total)
    del out
    want_m = 0
    step = 1 << 28
    for i in range(0, N, step):
        e = (y[i:i + step].to(torch.int32) >> 7) & 0xFF
        want_m += int((~member[e.long()]).sum().item())
    assert m == want_m
    got = y[idx].cpu().numpy().view(np.uint16)
    del y
    torch.cuda.empty_cache()
    assert np.array_equal(got, oracle.sum_words(rows))
    say("reduce_k checked")


@pytest.mark.parametrize("fmt,kept", [("s15", 15), ("z7", 7), ("t8", 8)])
def test_maximum_size_ablation_formats(fmt, kept):
    """The ablation formats at n = 2^32 - 1 uniformly random words: the
    values outside the first `kept` codebook exponents (escapes or
    zero-points) number more than 2^31. Checked: M against a count on the
    device and the bit-exact round trip."""
    say(f"{fmt} n={N} C={C}: generating uniform random words on the device")
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    x = torch.randint(-32768, 32768, (N,), dtype=torch.int16, device=DEV, generator=g)
    ocb = oracle.calibrate(x[: 1 << 20].cpu().numpy().view(np.uint16))
    cb = uzip.codebook_from_hist(ocb.hist)
    member = torch.zeros(256, dtype=torch.bool, device=DEV)
    member[torch.from_numpy(ocb.dec[:kept].astype(np.int64)).to(DEV)] = True
    enc = getattr(uzip, f"{fmt}_encode")
    dec = getattr(uzip, f"{fmt}_decode")
    say("encode")
    out = enc(x, cb, C)
    total, m = uzip.stream_bytes(out)
    say(f"M={m} total={total}")
    want_m = 0
    step = 1 << 28
    for i in range(0, N, step):
        e = (x[i:i + step].to(torch.int32) >> 7) & 0xFF
        want_m += int((~member[e.long()]).sum().item())
    assert m == want_m
    assert (1 << 31) < m < (1 << 32)
    say("decode")
    y = dec(out, cb, N, C, in_bytes=total)
    del out
    ok = torch.equal(y, x)
    del x, y
    torch.cuda.empty_cache()
    assert ok
    say("round trip bit-exact")
