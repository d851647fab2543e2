"""Escape placement across every per-tile escape count regime.

The placement writes a tile's escapes either one per lane (light tiles) or
as shifted 16-byte blocks from a position list or an escape bitmap (heavier
tiles), and neighbouring tiles share the 16-byte blocks at their edges. Here
consecutive 8192-value tiles carry escape counts on both sides of each
boundary (0, 1, 63-65, 127-130, 255-257, 511-513, 1053-1055 where the
exponent copy's first round is loaded ahead, a few thousand, all), in
mixed order and with the escapes spread out, bunched at the tile's start or
bunched at its end, plus a ragged last tile. Each placement wave writes the
chunk offsets of a run of 16 consecutive tiles and the escapes of those with
at most 64; heavier tiles are placed by waves of their own, so runs mix both
kinds, and with `pad` escape-free tiles added most runs hold light tiles
only. The streams must equal the oracle's byte for byte and decode to the
input, for the BF16 format, the Top-15 + sentinel format (no position array)
and the FP8 E5M2 format.
"""
import numpy as np
import pytest
import torch

import oracle
from lossless_bf16_tensor_amd import uzip

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TILE = 8192
COUNTS = [0, 1, 2, 63, 64, 65, 127, 128, 129, 130, 1, 255, 256, 257, 511, 512, 513, 128, 129, 0,
          1000, 64, 8192, 127, 3, 129, 4096, 128, 65, 512, 513, 7, 1053, 1054, 1055, 5, 1054, 2047, 2048]
LAST = (5000, 100)             # the ragged last tile: values, escapes


PADS = [0, 300]                # escape-free tiles added


def escape_mask(seed, pad=0):
    """A boolean mask over the whole input with COUNTS[i] escapes in tile i,
    then `pad` tiles without escapes and the ragged last tile."""
    rng = np.random.default_rng(seed)
    counts = COUNTS + [0] * pad
    n = TILE * len(counts) + LAST[0]
    mask = np.zeros(n, dtype=bool)
    for i, c in enumerate(counts + [LAST[1]]):
        size = TILE if i < len(counts) else LAST[0]
        t0 = i * TILE
        where = i % 3                              # spread, at the start, at the end
        if where == 0:
            idx = rng.choice(size, c, replace=False)
        elif where == 1:
            idx = np.arange(c)
        else:
            idx = np.arange(size - c, size)
        mask[t0 + idx] = True
    return mask


def bf16_input(seed, k=16, pad=0):
    """Words whose exponents are 120..120+k-1 (the codebook's) except at the
    mask's escapes (exponents 200..215)."""
    rng = np.random.default_rng(seed)
    mask = escape_mask(seed, pad)
    n = mask.size
    sm = rng.integers(0, 256, n).astype(np.uint16)
    e = np.where(mask, rng.integers(200, 216, n), rng.integers(120, 120 + k, n)).astype(np.uint16)
    x = ((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F)
    hist = np.zeros(256, np.uint64)
    hist[120:136] = np.arange(16, 0, -1, dtype=np.uint64) * 100
    return x.astype(np.uint16), hist, int(mask.sum())


def to_dev(x_np, dtype=np.int16):
    return torch.from_numpy(np.ascontiguousarray(x_np).view(dtype)).to(DEV)


def compare(got, want, label):
    assert got.size == want.size, f"{label}: size {got.size} != {want.size}"
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        pytest.fail(f"{label}: {bad.size} bytes differ, first at {bad[:8].tolist()}")


@pytest.mark.parametrize("pad", PADS)
@pytest.mark.parametrize("C", [64, 1024, 8192, 65536])
def test_bf16_escape_counts(C, pad):
    x, hist, m_want = bf16_input(C, pad=pad)
    ocb = oracle.top16(hist)
    cb = uzip.codebook_from_hist(hist)
    buf = uzip.encode(to_dev(x), cb, C)
    total, m = uzip.stream_bytes(buf)
    assert m == m_want
    compare(buf[:total].cpu().numpy(), oracle.encode(x, C, ocb.dec), f"bf16 C={C}")
    y = uzip.decode(buf, cb, x.size, C, in_bytes=total).cpu().numpy().view(np.uint16)
    assert np.array_equal(y, x)


@pytest.mark.parametrize("pad", PADS)
@pytest.mark.parametrize("C", [64, 1024, 4096])      # the format's largest chunk is 4096
def test_sentinel_escape_counts(C, pad):
    x, hist, m_want = bf16_input(C + 1, k=15, pad=pad)   # the sentinel format codes 15 exponents
    ocb = oracle.calibrate(np.repeat(np.array([oracle.merge(0, e) for e in range(120, 136)], np.uint16),
                                     np.arange(16, 0, -1)))
    cb = uzip.codebook_from_hist(ocb.hist)
    buf = uzip.s15_encode(to_dev(x), cb, C)
    total, m = uzip.stream_bytes(buf)
    assert m == m_want
    compare(buf[:total].cpu().numpy(), oracle.s15_encode(x, C, ocb.dec), f"s15 C={C}")
    y = uzip.s15_decode(buf, cb, x.size, C, in_bytes=total).cpu().numpy().view(np.uint16)
    assert np.array_equal(y, x)


@pytest.mark.parametrize("pad", PADS)
@pytest.mark.parametrize("C", [64, 1024, 8192])
def test_fp8_escape_counts(C, pad):
    rng = np.random.default_rng(C + 2)
    mask = escape_mask(C + 2, pad)
    n = mask.size
    a = rng.integers(0, 8, n)
    e = np.where(mask, rng.integers(16, 32, n), rng.integers(0, 16, n))
    # the merge for every value, vectorised: sign (bit 2 of a) to bit 7,
    # the exponent to bits 2..6, the mantissa (bits 0..1 of a) to bits 0..1
    x = (((a >> 2) & 1) << 7 | (e & 0x1F) << 2 | (a & 3)).astype(np.uint8)
    assert all(int(x[i]) == oracle.fp8_merge(int(a[i]), int(e[i])) for i in range(64))
    ocb = oracle.fp8_calibrate(np.repeat(np.array([oracle.fp8_merge(0, k) for k in range(16)], np.uint8),
                                         np.arange(16, 0, -1)))
    cb = uzip.codebook_from_hist(ocb.hist)
    buf = uzip.fp8_encode(torch.from_numpy(x).to(DEV), cb, C)
    total, m = uzip.stream_bytes(buf)
    assert m == int(mask.sum())
    compare(buf[:total].cpu().numpy(), oracle.fp8_encode(x, C, ocb.dec), f"fp8 C={C}")
    y = uzip.fp8_decode(buf, cb, n, C, in_bytes=total).cpu().numpy()
    assert np.array_equal(y, x)


def dirty(nbytes, fill, seed):
    """A device buffer of nbytes holding `fill` in every byte, or random bytes
    when fill is None."""
    if fill is None:
        rng = np.random.default_rng(seed)
        return torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).to(DEV)
    return torch.full((nbytes,), fill, dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("fill", [0x00, 0xFF, None])
def test_dirty_workspace(fill):
    # The placement loads staged bytes past a tile's escapes (each light
    # tile's entry `lane`, whole 16-byte blocks at a list's end, the copy's
    # first round of exponent blocks) but never uses them: streams written
    # with a workspace and output buffer full of other bytes equal the
    # oracle's, for encode and both reduces.
    C = 1024
    x, hist, _ = bf16_input(21, pad=40)
    x2, _, _ = bf16_input(22, pad=40)
    n = x.size
    ocb = oracle.top16(hist)
    cb = uzip.codebook_from_hist(hist)
    wsb = uzip.workspace_bytes(n, C)
    cap = uzip.max_bytes(n, C)
    a = uzip.encode(to_dev(x), cb, C, out=dirty(cap, fill, 1), ws=dirty(wsb, fill, 2))
    ta, _ = uzip.stream_bytes(a)
    oa = oracle.encode(x, C, ocb.dec)
    compare(a[:ta].cpu().numpy(), oa, f"encode fill={fill}")
    b = uzip.encode(to_dev(x2), cb, C, out=dirty(cap, fill, 3), ws=dirty(wsb, fill, 4))
    tb, _ = uzip.stream_bytes(b)
    ob = oracle.encode(x2, C, ocb.dec)
    compare(b[:tb].cpu().numpy(), ob, f"encode 2 fill={fill}")
    r = uzip.reduce_add(a[:ta], b[:tb], cb, n, C, out=dirty(cap, fill, 5), ws=dirty(wsb, fill, 6))
    tr, _ = uzip.stream_bytes(r)
    compare(r[:tr].cpu().numpy(), oracle.reduce_add(oa, ob, n, C, ocb.dec), f"reduce_add fill={fill}")
    rk = uzip.reduce_k([a[:ta], b[:tb], a[:ta]], cb, n, C, out=dirty(cap, fill, 7), ws=dirty(wsb, fill, 8))
    tk, _ = uzip.stream_bytes(rk)
    compare(rk[:tk].cpu().numpy(), oracle.reduce_k([oa, ob, oa], n, C, ocb.dec), f"reduce_k fill={fill}")
