"""Seeded random parity sweep over sizes, chunk sizes and escape layouts.

Each case draws n (log-uniform up to 3 million), a chunk size (a power of two
in [64, 65536]) and, per 8192-word tile, an escape density from {0, 0.1 %,
1 %, 5 %, 20 %, all} (escapes include zeros, subnormals, infinities and
NaNs, so the reduces meet them too), so that light and heavy tiles sit side
by side in the placement's runs of consecutive tiles. Every format the library encodes is checked against the oracle
byte for byte (BF16, Top-15 + sentinel and Top-7 + zero-point where the chunk
size allows them, Top-8 3-bit, FP8 E5M2), with the decode equal to the input;
every fifth case adds online calibration (whole input or a block sample),
every third the fused reduce of two such inputs and every fourth the k-input
reduce of up to four.
"""
import numpy as np
import pytest
import torch

import oracle
from lossless_bf16_tensor_amd import uzip

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TILE = 8192
DENSITIES = np.array([0.0, 0.001, 0.01, 0.05, 0.2, 1.0])
CASES = list(range(160))


def escape_mask(rng, n):
    nt = (n + TILE - 1) // TILE
    dens = rng.choice(DENSITIES, size=nt, p=[0.3, 0.2, 0.2, 0.15, 0.1, 0.05])
    u = rng.random(n)
    return u < np.repeat(dens, TILE)[:n]


# escape exponents: the codebook's neighbours, zeros and subnormals (0), the
# largest finite binade (254), infinities and NaNs (255), and far ones
ESCAPE_EXPONENTS = np.array([0, 1, 118, 119, 136, 137, 254, 255] + list(range(200, 216)))


def bf16_words(rng, n, mask):
    """Exponents 120..135 (weighted towards 120) off the mask, escape
    exponents on it."""
    e_in = 120 + np.minimum(rng.geometric(0.3, n) - 1, 15)
    e = np.where(mask, rng.choice(ESCAPE_EXPONENTS, n), e_in).astype(np.uint16)
    a = rng.integers(0, 256, n).astype(np.uint16)
    return (((a & 0x80) << 8) | (e << 7) | (a & 0x7F)).astype(np.uint16)


def bf16_codebook():
    hist = np.zeros(256, np.uint64)
    hist[120:136] = np.arange(16, 0, -1, dtype=np.uint64) * 1000
    return oracle.top16(hist), uzip.codebook_from_hist(hist)


def fp8_bytes(rng, n, mask):
    e = np.where(mask, rng.integers(16, 32, n), np.minimum(rng.geometric(0.3, n) - 1, 15))
    a = rng.integers(0, 8, n)
    return (((a >> 2) & 1) << 7 | (e & 0x1F) << 2 | (a & 3)).astype(np.uint8)


def fp8_codebook():
    calib = np.repeat(np.array([oracle.fp8_merge(0, k) for k in range(16)], np.uint8), np.arange(16, 0, -1))
    ocb = oracle.fp8_calibrate(calib)
    return ocb, uzip.codebook_from_hist(ocb.hist)


def compare(got, want, label):
    assert got.size == want.size, f"{label}: size {got.size} != {want.size}"
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        pytest.fail(f"{label}: {bad.size} bytes differ, first at {bad[:8].tolist()}")


def words_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV)


def check_words(fmt, x, C, ocb, cb, label):
    enc, dec, oenc = {
        "bf16": (uzip.encode, uzip.decode, oracle.encode),
        "s15": (uzip.s15_encode, uzip.s15_decode, oracle.s15_encode),
        "z7": (uzip.z7_encode, uzip.z7_decode, oracle.z7_encode),
        "t8": (uzip.t8_encode, uzip.t8_decode, oracle.t8_encode),
    }[fmt]
    buf = enc(words_dev(x), cb, C)
    total, _ = uzip.stream_bytes(buf)
    compare(buf[:total].cpu().numpy(), oenc(x, C, ocb.dec), f"{label} {fmt}")
    y = dec(buf, cb, x.size, C, in_bytes=total).cpu().numpy().view(np.uint16)
    assert np.array_equal(y, x), f"{label} {fmt}: decode differs"
    return buf, total


@pytest.mark.parametrize("case", CASES)
def test_random_case(case):
    rng = np.random.default_rng(7000 + case)
    n = int(10 ** rng.uniform(0, np.log10(3_000_000)))
    C = int(2 ** rng.integers(6, 17))
    label = f"case {case}: n={n} C={C}"
    ocb, cb = bf16_codebook()
    x = bf16_words(rng, n, escape_mask(rng, n))
    buf, total = check_words("bf16", x, C, ocb, cb, label)
    check_words("t8", x, C, ocb, cb, label)
    if C <= 4096:
        check_words("s15", x, C, ocb, cb, label)
        check_words("z7", x, C, ocb, cb, label)
    # FP8 E5M2 over the same layout of escapes
    o8, c8 = fp8_codebook()
    x8 = fp8_bytes(rng, n, escape_mask(rng, n))
    b8 = uzip.fp8_encode(torch.from_numpy(x8).to(DEV), c8, C)
    t8, _ = uzip.stream_bytes(b8)
    compare(b8[:t8].cpu().numpy(), oracle.fp8_encode(x8, C, o8.dec), f"{label} fp8")
    assert np.array_equal(uzip.fp8_decode(b8, c8, n, C, in_bytes=t8).cpu().numpy(), x8), f"{label} fp8 decode"
    if case % 5 == 0:
        # online calibration: the whole input, or the first `sample` words of every `block`
        if rng.random() < 0.5:
            block = sample = 0
            ocal = x
        else:
            block = int(8 * 2 ** rng.integers(0, 15))
            sample = int(8 * rng.integers(1, block // 8 + 1))
            ocal = oracle.sample_words(x, block, sample)
        bo = uzip.encode_online(words_dev(x), C, block, sample)
        to, _ = uzip.stream_bytes(bo)
        compare(bo[:to].cpu().numpy(), oracle.encode(x, C, oracle.calibrate(ocal).dec),
                f"{label} online block={block} sample={sample}")
        rcb = uzip.codebook_from_dec(uzip.parse_header(bo[:256].cpu().numpy().tobytes())["dec"])
        y = uzip.decode(bo, rcb, n, C, in_bytes=to).cpu().numpy().view(np.uint16)
        assert np.array_equal(y, x), f"{label} online decode"
    if case % 3 == 0:
        xb = bf16_words(rng, n, escape_mask(rng, n))
        bb = uzip.encode(words_dev(xb), cb, C)
        tb, _ = uzip.stream_bytes(bb)
        r = uzip.reduce_add(buf[:total], bb[:tb], cb, n, C)
        tr, _ = uzip.stream_bytes(r)
        want = oracle.reduce_add(oracle.encode(x, C, ocb.dec), oracle.encode(xb, C, ocb.dec), n, C, ocb.dec)
        compare(r[:tr].cpu().numpy(), want, f"{label} reduce_add")
    if case % 4 == 0:
        k = int(rng.integers(1, 5))
        xs = [bf16_words(rng, n, escape_mask(rng, n)) for _ in range(k)]
        streams, ostreams = [], []
        for xi in xs:
            bi = uzip.encode(words_dev(xi), cb, C)
            ti, _ = uzip.stream_bytes(bi)
            streams.append(bi[:ti])
            ostreams.append(oracle.encode(xi, C, ocb.dec))
        r = uzip.reduce_k(streams, cb, n, C)
        tr, _ = uzip.stream_bytes(r)
        compare(r[:tr].cpu().numpy(), oracle.reduce_k(ostreams, n, C, ocb.dec), f"{label} reduce_k k={k}")
