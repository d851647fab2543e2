"""GPU parity: the HIP path against the CPU oracle, bit for bit.

Every stream the GPU writes must equal the oracle's byte for byte, decoded
tensors must equal the input word for word (0 ulp), and the fused reduce must
equal the oracle's decode-add-reencode. All calls go through the C-ABI
(ctypes binding). Inputs are the seeded workloads of the five configurations
(full sizes included) plus exhaustive and ragged cases.
"""
import functools

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


@functools.lru_cache(maxsize=None)
def workload(k, small=False):
    return workloads.config(k, small=small)


def gpu_codebook(*calib):
    hist = None
    for c in calib:
        hist = uzip.histogram(to_dev(c), hist)
    return uzip.codebook_from_hist(hist.cpu().numpy().astype(np.uint64)), hist


def check_encode(x_np, C, cb, ocb, label):
    """GPU stream == oracle stream; GPU decode (both variants) == x."""
    x = to_dev(x_np)
    buf = uzip.encode(x, cb, C)
    total, m = uzip.stream_bytes(buf)
    want = oracle.encode(x_np, C, ocb.dec)
    got = buf[:total].cpu().numpy()
    assert total == want.size, f"{label}: size {total} != {want.size}"
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        pytest.fail(f"{label}: {bad.size} bytes differ, first at {bad[:8].tolist()}")
    for sep in (False, True):
        y = uzip.decode(buf, cb, x_np.size, C, in_bytes=total, separate_patch=sep)
        yh = host_words(y)
        if not np.array_equal(yh, x_np):
            bad = np.nonzero(yh != x_np)[0]
            pytest.fail(f"{label} decode(separate_patch={sep}): {bad.size} words differ, first {bad[:8].tolist()}")
    return buf, total, m


def test_histogram_matches_oracle():
    for k in (1, 2, 4):
        w = workload(k)
        _, hist = gpu_codebook(w.calib)
        assert np.array_equal(hist.cpu().numpy().astype(np.uint64), oracle.histogram(w.calib)), k
    x = workloads.random_words(8 * 1000 + 5, 3)            # ragged tail
    _, hist = gpu_codebook(x)
    assert np.array_equal(hist.cpu().numpy().astype(np.uint64), oracle.histogram(x))


def test_calibrate_matches_oracle_codebook():
    w = workload(1)
    cb = uzip.calibrate(to_dev(w.calib))
    ocb = oracle.calibrate(w.calib)
    assert list(cb.dec) == ocb.dec.tolist()
    assert list(cb.enc) == ocb.enc.tolist() and list(cb.member) == ocb.member.tolist()


@pytest.mark.parametrize("C", [64, 256, 1024, 4096, 65536])
def test_all_words_every_chunk(C):
    x = workloads.all_patterns(seed=C)
    for calib in (x, workloads.bf16_bits(np.random.default_rng(0).standard_normal(50000))):
        cb, _ = gpu_codebook(calib)
        ocb = oracle.calibrate(calib)
        check_encode(x, C, cb, ocb, f"all-words C={C}")


@pytest.mark.parametrize("n", [1, 2, 3, 7, 8, 9, 15, 16, 17, 63, 64, 65, 1023, 2047, 8191, 8192, 8193,
                               16385, 3 * 65536 + 17, 1 << 18])
def test_ragged_sizes(n):
    x = workloads.random_words(n, seed=n)
    calib = workloads.bf16_bits(np.random.default_rng(1).standard_normal(50000))
    cb, _ = gpu_codebook(calib)
    ocb = oracle.calibrate(calib)
    for C in (64, 1024, 65536):
        check_encode(x, C, cb, ocb, f"random n={n} C={C}")


def test_dense_escapes_everywhere():
    # codebook disjoint from the data: every word is an escape (M = n)
    rng = np.random.default_rng(9)
    x = (rng.integers(0, 256, 100003).astype(np.uint16) & 0x807F) | (np.uint16(200) << 7)
    h = np.zeros(256, np.uint64)
    h[0:16] = 1
    cb = uzip.codebook_from_hist(h)
    ocb = oracle.top16(h)
    for C in (64, 256, 8192, 65536):
        _, _, m = check_encode(x, C, cb, ocb, f"all-escape C={C}")
        assert m == x.size


def test_no_escapes():
    w = workload(1)
    ocb = oracle.calibrate(w.calib)
    e = ocb.dec[np.random.default_rng(2).integers(0, 16, 300000)].astype(np.uint16)
    a = np.random.default_rng(3).integers(0, 256, 300000).astype(np.uint16)
    x = ((a & 0x80) << 8) | (e << 7) | (a & 0x7F)
    cb = uzip.codebook_from_hist(ocb.hist)
    _, _, m = check_encode(x, 1024, cb, ocb, "no-escape")
    assert m == 0


def test_config1_full():
    w = workload(1)
    cb, _ = gpu_codebook(w.calib)
    ocb = oracle.calibrate(w.calib)
    assert list(cb.dec) == ocb.dec.tolist()
    check_encode(w.x, 1024, cb, ocb, "config 1")


def test_config2_full():
    w = workload(2)
    cb, _ = gpu_codebook(w.calib)
    ocb = oracle.calibrate(w.calib)
    check_encode(w.x, 1024, cb, ocb, "config 2")


def test_config3_small():
    w = workload(3, small=True)
    cb, _ = gpu_codebook(w.calib)
    ocb = oracle.calibrate(w.calib)
    check_encode(w.x, 1024, cb, ocb, "config 3 small")


def test_config4_full_three_chunks():
    w = workload(4)
    cb, _ = gpu_codebook(w.calib)
    ocb = oracle.calibrate(w.calib)
    dense = None
    for C in w.chunks:
        buf, total, m = check_encode(w.x, C, cb, ocb, f"config 4 C={C}")
        sec = oracle.sections(buf[:total].cpu().numpy())
        # ratio formula: payload N + N/2 + 3M
        assert sec["sm"].size + sec["codes"].size + 3 * sec["m"] == oracle.payload_bytes(w.x.size, m)
        if dense is None:
            dense = (sec["sm"].copy(), sec["codes"].copy(), m)
        else:
            assert np.array_equal(sec["sm"], dense[0]) and np.array_equal(sec["codes"], dense[1])
            assert m == dense[2]


def test_config3_full():
    w = workload(3)
    cb, _ = gpu_codebook(w.calib)
    ocb = oracle.calibrate(w.calib)
    assert list(cb.dec) == ocb.dec.tolist()
    check_encode(w.x, 1024, cb, ocb, "config 3 (2^28)")


def test_encode_is_deterministic_and_leaves_tail_bytes():
    w = workload(2)
    cb, _ = gpu_codebook(w.calib)
    x = to_dev(w.x)
    cap = uzip.max_bytes(w.x.size, 1024)
    out1 = torch.full((cap,), 0xA5, dtype=torch.uint8, device=DEV)
    out2 = torch.full((cap,), 0x5A, dtype=torch.uint8, device=DEV)
    uzip.encode(x, cb, 1024, out=out1)
    uzip.encode(x, cb, 1024, out=out2)
    total, _ = uzip.stream_bytes(out1)
    assert torch.equal(out1[:total], out2[:total])
    assert bool((out1[total:] == 0xA5).all()) and bool((out2[total:] == 0x5A).all())
    assert uzip.validate(out1, cb) == 0


# --------------------------------------------------------------- reduce ----
def check_reduce(a_np, b_np, C, cb, ocb, label):
    A = uzip.encode(to_dev(a_np), cb, C)
    B = uzip.encode(to_dev(b_np), cb, C)
    ta, _ = uzip.stream_bytes(A)
    tb, _ = uzip.stream_bytes(B)
    R = uzip.reduce_add(A[:ta], B[:tb], cb, a_np.size, C)
    tr, _ = uzip.stream_bytes(R)
    sa = oracle.encode(a_np, C, ocb.dec)
    sb = oracle.encode(b_np, C, ocb.dec)
    want = oracle.reduce_add(sa, sb, a_np.size, C, ocb.dec)
    got = R[:tr].cpu().numpy()
    assert tr == want.size, f"{label}: size {tr} != {want.size}"
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        pytest.fail(f"{label}: {bad.size} bytes differ, first at {bad[:8].tolist()}")
    return R, tr


def test_reduce_special_values():
    # pairs chosen for rounding ties, subnormal sums, overflow, signed zeros,
    # infinities and NaNs, tiled to cover several tiles and a ragged tail
    edge = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x3F80, 0xBF80,
                     0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0xFFC1, 0x3F81, 0x3B80,
                     0x4000, 0x0100, 0x7F00, 0x3380, 0x3F7F], dtype=np.uint16)
    aa, bb = np.meshgrid(edge, edge)
    a = np.tile(aa.reshape(-1), 40)
    b = np.tile(bb.reshape(-1), 40)
    rng = np.random.default_rng(4)
    extra_a = rng.integers(0, 65536, 30011).astype(np.uint16)
    extra_b = (extra_a & 0xFF80) ^ rng.integers(0, 0x180, 30011).astype(np.uint16)
    a = np.concatenate([a, extra_a])
    b = np.concatenate([b, extra_b])
    ocb = oracle.calibrate(a, b)
    cb = uzip.codebook_from_hist(ocb.hist)
    for C in (64, 1024, 65536):
        R, tr = check_reduce(a, b, C, cb, ocb, f"reduce edge C={C}")
        y = host_words(uzip.decode(R, cb, a.size, C, in_bytes=tr))
        assert np.array_equal(y, oracle.add_words(a, b))


def test_reduce_config5_small():
    w = workload(5, small=True)
    A, B = w.x
    ocb = oracle.calibrate(A, B)
    cb, _ = gpu_codebook(A, B)
    assert list(cb.dec) == ocb.dec.tolist()
    check_reduce(A, B, 1024, cb, ocb, "config 5 small")


@pytest.mark.timeout(900)
def test_config5_full_reduce():
    w = workload(5)
    A, B = w.x
    print("config 5: inputs ready", flush=True)
    cb, _ = gpu_codebook(A, B)
    ocb = oracle.calibrate(A, B)
    assert list(cb.dec) == ocb.dec.tolist()
    check_encode(A, 1024, cb, ocb, "config 5 A")
    check_encode(B, 1024, cb, ocb, "config 5 B")
    print("config 5: inputs encoded", flush=True)
    check_reduce(A, B, 1024, cb, ocb, "config 5 reduce (2 x 2^29)")


def test_worked_example_stream():
    # the stream worked out by hand from the stream layout
    # (tests/golden/stream_worked_example.txt), through the C-ABI
    from test_oracle_format import CHUNK, WORDS, golden_hist, golden_stream
    cb = uzip.codebook_from_hist(golden_hist())
    want = golden_stream()
    buf = uzip.encode(to_dev(WORDS), cb, CHUNK)
    total, m = uzip.stream_bytes(buf)
    assert (total, m) == (want.size, 1)
    assert np.array_equal(buf[:total].cpu().numpy(), want)
    y = uzip.decode(buf, cb, WORDS.size, CHUNK, in_bytes=total).cpu().numpy().view(np.uint16)
    assert np.array_equal(y, WORDS)
    assert uzip.validate(buf[:total], cb) == 0


@pytest.mark.parametrize("fmt", ["s15", "z7"])
def test_worked_example_ablation_streams(fmt):
    # the Top-15 + sentinel and Top-7 + zero-point streams worked out by hand
    from test_oracle_format import CHUNK, GOLDEN_S15, GOLDEN_Z7, WORDS, golden_hist, golden_stream
    cb = uzip.codebook_from_hist(golden_hist())
    want = golden_stream({"s15": GOLDEN_S15, "z7": GOLDEN_Z7}[fmt])
    buf = getattr(uzip, f"{fmt}_encode")(to_dev(WORDS), cb, CHUNK)
    total, m = uzip.stream_bytes(buf)
    assert (total, m) == (want.size, 1)
    assert np.array_equal(buf[:total].cpu().numpy(), want)
    y = getattr(uzip, f"{fmt}_decode")(buf, cb, WORDS.size, CHUNK, in_bytes=total).cpu().numpy().view(np.uint16)
    assert np.array_equal(y, WORDS)


def test_worked_example_reduce():
    # the fused reduce worked out by hand (tests/golden/stream_reduce_worked_example.txt),
    # through both reduce entry points
    from test_oracle_format import CHUNK, GOLDEN_REDUCE, WORDS, WORDS_B, golden_hist, golden_stream
    cb = uzip.codebook_from_hist(golden_hist())
    want = golden_stream(GOLDEN_REDUCE)
    a = uzip.encode(to_dev(WORDS), cb, CHUNK)
    b = uzip.encode(to_dev(WORDS_B), cb, CHUNK)
    ta, _ = uzip.stream_bytes(a)
    tb, _ = uzip.stream_bytes(b)
    for r in (uzip.reduce_add(a[:ta], b[:tb], cb, WORDS.size, CHUNK),
              uzip.reduce_k([a[:ta], b[:tb]], cb, WORDS.size, CHUNK)):
        total, m = uzip.stream_bytes(r)
        assert (total, m) == (want.size, 1)
        assert np.array_equal(r[:total].cpu().numpy(), want)
