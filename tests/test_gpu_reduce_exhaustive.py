"""The fused reduce's arithmetic on every pair of BF16 words.

All 2^32 (a, b) pairs go through uzip_reduce_add, 2^28 pairs per call: a
stream of the a words and a stream of the b words (every word, in order) are
encoded, reduced, and the result decoded. Each decoded sum must equal the
oracle's add word for word: one IEEE binary32 add (round to nearest even,
subnormals kept), then round half to even to BF16, a NaN sum becoming 0x7FC0
(the reduce of "UCCL-Zip: Lossless Compression Supercharged GPU
Communication", section 3.4, with the precision of the benchmark spec). The
oracle's add is itself pinned against exact rationals and float64 in
tests/test_oracle_reduce.py. This covers the kernel's hardware BF16 rounding
on every input the reduce can meet, not a sample."""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import oracle
from lossless_bf16_tensor_amd import uzip

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
C = 1024
SLICE_A = 4096                       # a values per call: 4096 x 65536 = 2^28 pairs


def oracle_add_parallel(a, b, pool, parts=8):
    out = np.empty(a.size, dtype=np.uint16)
    step = (a.size + parts - 1) // parts

    def one(i):
        out[i:i + step] = oracle.add_words(a[i:i + step], b[i:i + step])

    list(pool.map(one, range(0, a.size, step)))
    return out


def test_reduce_every_bf16_pair():
    n = SLICE_A * 65536
    b_np = np.tile(np.arange(65536, dtype=np.uint16), SLICE_A)
    # a codebook of the 16 most common exponents of normal numbers near 1:
    # most words of these inputs are escapes, which the reduce must patch
    hist = np.zeros(256, dtype=np.uint64)
    hist[120:136] = np.arange(16, 0, -1, dtype=np.uint64) * 1000
    cb = uzip.codebook_from_hist(hist)
    ws = torch.empty(uzip.workspace_bytes(n, C), dtype=torch.uint8, device=DEV)
    sb = uzip.encode(torch.from_numpy(b_np.view(np.int16)).to(DEV), cb, C, ws=ws)
    tb, _ = uzip.stream_bytes(sb)
    sa = torch.empty_like(sb)
    sr = torch.empty_like(sb)
    y = torch.empty(n, dtype=torch.int16, device=DEV)
    bad_total = 0
    with cf.ThreadPoolExecutor(8) as pool:
        for s in range(65536 // SLICE_A):
            a_np = np.repeat(np.arange(s * SLICE_A, (s + 1) * SLICE_A, dtype=np.uint16), 65536)
            uzip.encode(torch.from_numpy(a_np.view(np.int16)).to(DEV), cb, C, out=sa, ws=ws)
            ta, _ = uzip.stream_bytes(sa)
            uzip.reduce_add(sa[:ta], sb[:tb], cb, n, C, out=sr, ws=ws)
            tr, _ = uzip.stream_bytes(sr)
            uzip.decode(sr, cb, n, C, out=y, in_bytes=tr)
            got = y.cpu().numpy().view(np.uint16)
            want = oracle_add_parallel(a_np, b_np, pool)
            bad = np.nonzero(got != want)[0]
            if bad.size:
                i = int(bad[0])
                pytest.fail(f"slice {s}: {bad.size} sums differ, first a=0x{a_np[i]:04x} b=0x{b_np[i]:04x}: "
                            f"got 0x{got[i]:04x}, want 0x{want[i]:04x}")
            bad_total += bad.size
    assert bad_total == 0
