"""The stream layout pinned by a stream worked out by hand
(tests/golden/stream_worked_example.txt): five words, one escape, chunk 64.
The oracle's stream must equal it byte for byte, and its decode must return
the words. The GPU encode is checked against the same bytes in
tests/test_gpu_parity.py."""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "stream_worked_example.txt")
WORDS = np.array([0x3F80, 0x4000, 0xBF80, 0x7F80, 0x0001], dtype=np.uint16)
CHUNK = 64


def golden_stream():
    total, runs = None, []
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        head, *rest = line.split()
        if head == "total":
            total = int(rest[0])
        else:
            runs.append((int(head), bytes(int(b, 16) for b in rest)))
    s = np.zeros(total, dtype=np.uint8)
    for off, b in runs:
        s[off:off + len(b)] = np.frombuffer(b, dtype=np.uint8)
    return s


def golden_hist():
    h = np.zeros(256, dtype=np.uint64)
    h[127], h[128], h[0] = 10, 5, 3
    return h


def test_codebook_of_the_worked_example():
    cb = oracle.top16(golden_hist())
    assert cb.dec.tolist() == [127, 128, 0] + list(range(1, 14))


def test_oracle_stream_equals_the_worked_example():
    cb = oracle.top16(golden_hist())
    got = oracle.encode(WORDS, CHUNK, cb.dec)
    want = golden_stream()
    assert got.size == want.size == 1281
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:16].tolist()
    assert np.array_equal(oracle.decode(want, WORDS.size, CHUNK, cb.dec), WORDS)
    assert oracle.validate(want, cb.dec) == 0
