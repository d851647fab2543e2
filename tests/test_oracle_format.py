"""The stream layouts pinned by streams worked out by hand, chunk 64: five
BF16 words with one escape (tests/golden/stream_worked_example.txt), the
same words in the Top-15 + sentinel and Top-7 + zero-point formats
(stream_s15_worked_example.txt, stream_z7_worked_example.txt), five FP8
E5M2 values with one escape (stream_fp8_worked_example.txt), and the fused
reduce of the five BF16 words with five ones (stream_reduce_worked_example.txt).
The oracle's streams must equal them byte for byte and its decodes return
the inputs; the GPU paths are checked against the same bytes in
tests/test_gpu_parity.py and tests/test_gpu_fp8.py."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "stream_worked_example.txt")
GOLDEN_FP8 = os.path.join(os.path.dirname(__file__), "golden", "stream_fp8_worked_example.txt")
GOLDEN_S15 = os.path.join(os.path.dirname(__file__), "golden", "stream_s15_worked_example.txt")
GOLDEN_Z7 = os.path.join(os.path.dirname(__file__), "golden", "stream_z7_worked_example.txt")
GOLDEN_REDUCE = os.path.join(os.path.dirname(__file__), "golden", "stream_reduce_worked_example.txt")
WORDS_B = np.full(5, 0x3F80, dtype=np.uint16)
WORDS = np.array([0x3F80, 0x4000, 0xBF80, 0x7F80, 0x0001], dtype=np.uint16)
BYTES_FP8 = np.array([0x3C, 0x40, 0xBC, 0x7C, 0x01], dtype=np.uint8)
CHUNK = 64


def golden_stream(path=GOLDEN):
    total, runs = None, []
    for line in open(path):
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


def golden_hist_fp8():
    h = np.zeros(32, dtype=np.uint64)
    h[15], h[16], h[0] = 10, 5, 3
    return h


def test_oracle_fp8_stream_equals_the_worked_example():
    calib = np.repeat(np.array([0x3C, 0x40, 0x00], dtype=np.uint8), [10, 5, 3])   # e 15, 16, 0
    cb = oracle.fp8_calibrate(calib)
    assert np.array_equal(cb.hist[:32], golden_hist_fp8())
    assert cb.dec.tolist() == [15, 16, 0] + list(range(1, 14))
    got = oracle.fp8_encode(BYTES_FP8, CHUNK, cb.dec)
    want = golden_stream(GOLDEN_FP8)
    assert got.size == want.size == 1281
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:16].tolist()
    assert np.array_equal(oracle.fp8_decode(want, BYTES_FP8.size, CHUNK, cb.dec), BYTES_FP8)
    assert oracle.fp8_validate(want, cb.dec) == 0


@pytest.mark.parametrize("fmt,path", [("s15", GOLDEN_S15), ("z7", GOLDEN_Z7)])
def test_oracle_ablation_streams_equal_the_worked_examples(fmt, path):
    cb = oracle.top16(golden_hist())
    got = getattr(oracle, f"{fmt}_encode")(WORDS, CHUNK, cb.dec)
    want = golden_stream(path)
    assert got.size == want.size
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:16].tolist()
    assert np.array_equal(getattr(oracle, f"{fmt}_decode")(want, WORDS.size, CHUNK, cb.dec), WORDS)
    assert getattr(oracle, f"{fmt}_validate")(want, cb.dec) == 0


def test_oracle_reduce_equals_the_worked_example():
    cb = oracle.top16(golden_hist())
    sa, sb = oracle.encode(WORDS, CHUNK, cb.dec), oracle.encode(WORDS_B, CHUNK, cb.dec)
    want = golden_stream(GOLDEN_REDUCE)
    for got in (oracle.reduce_add(sa, sb, WORDS.size, CHUNK, cb.dec),
                oracle.reduce_k([sa, sb], WORDS.size, CHUNK, cb.dec)):
        assert got.size == want.size
        assert np.array_equal(got, want), np.nonzero(got != want)[0][:16].tolist()
    sums = oracle.decode(want, WORDS.size, CHUNK, cb.dec)
    assert sums.tolist() == [0x4000, 0x4040, 0x0000, 0x7F80, 0x3F80]

