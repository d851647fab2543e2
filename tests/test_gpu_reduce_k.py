"""GPU parity of the k-input fused reduce (uzip_reduce_k) against the oracle:
the output stream must equal the oracle's byte for byte. Inputs are encoded
by each side on its own (the oracle never sees a GPU-made stream)."""
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


def gpu_reduce_k(rows, C, cb):
    streams = [uzip.encode(to_dev(r), cb, C) for r in rows]
    sizes = [uzip.stream_bytes(s)[0] for s in streams]
    R = uzip.reduce_k([s[:t] for s, t in zip(streams, sizes)], cb, rows[0].size, C)
    tr, _ = uzip.stream_bytes(R)
    return R, tr, streams, sizes


def check_reduce_k(rows, C, cb, ocb, label):
    R, tr, _, _ = gpu_reduce_k(rows, C, cb)
    ostreams = [oracle.encode(r, C, ocb.dec) for r in rows]
    want = oracle.reduce_k(ostreams, rows[0].size, C, ocb.dec)
    got = R[:tr].cpu().numpy()
    assert tr == want.size, f"{label}: size {tr} != {want.size}"
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        pytest.fail(f"{label}: {bad.size} bytes differ, first at {bad[:8].tolist()}")
    return R, tr


def random_rows(k, n, seed):
    """BF16 words with exponents spread around 1.0, so that sums round and a
    few percent of the values (and sums) fall outside the codebook."""
    rng = np.random.default_rng(seed)
    e = np.clip(np.round(rng.normal(127, 4, (k, n))), 1, 254).astype(np.uint16)
    m = rng.integers(0, 128, (k, n)).astype(np.uint16)
    s = rng.integers(0, 2, (k, n)).astype(np.uint16)
    return [r for r in ((s << 15) | (e << 7) | m)]


def codebooks(rows):
    ocb = oracle.calibrate(*rows)
    return uzip.codebook_from_hist(ocb.hist), ocb


@pytest.mark.parametrize("k", [1, 2, 3, 5, 8, 16])
def test_reduce_k_matches_oracle(k):
    rows = random_rows(k, 50011, 100 + k)
    cb, ocb = codebooks(rows)
    check_reduce_k(rows, 1024, cb, ocb, f"k={k}")


@pytest.mark.parametrize("C", [64, 256, 4096, 65536])
def test_reduce_k_chunk_sizes(C):
    rows = random_rows(4, 70001, 7)
    cb, ocb = codebooks(rows)
    check_reduce_k(rows, C, cb, ocb, f"k=4 C={C}")


@pytest.mark.parametrize("n", [1, 7, 8, 9, 8191, 8192, 8193, 16385])
def test_reduce_k_ragged(n):
    rows = random_rows(3, n, 9)
    cb, ocb = codebooks(rows)
    check_reduce_k(rows, 1024, cb, ocb, f"k=3 n={n}")


def test_two_inputs_equal_the_pairwise_kernel():
    rows = random_rows(2, 100003, 21)
    cb, _ = codebooks(rows)
    R, tr, streams, sizes = gpu_reduce_k(rows, 1024, cb)
    P = uzip.reduce_add(streams[0][:sizes[0]], streams[1][:sizes[1]], cb, rows[0].size, 1024)
    tp, _ = uzip.stream_bytes(P)
    assert tr == tp and torch.equal(R[:tr], P[:tp])


def test_reduce_k_special_values():
    # every column of edge values in 3 inputs, plus the order-sensitive
    # column [1, 2^-8, 2^-24, 2^-24] and its reverse in 4 inputs
    edge = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x7F7F, 0xFF7F,
                     0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0x3F81, 0x3B80, 0x3380], dtype=np.uint16)
    g = np.stack(np.meshgrid(edge, edge, edge, indexing="ij")).reshape(3, -1)
    rows3 = [np.tile(g[i], 7) for i in range(3)]
    cb, ocb = codebooks(rows3)
    R, tr = check_reduce_k(rows3, 1024, cb, ocb, "edge k=3")
    y = host_words(uzip.decode(R, cb, rows3[0].size, 1024, in_bytes=tr))
    assert np.array_equal(y, oracle.sum_words(np.stack(rows3)))
    col = np.array([0x3F80, 0x3B80, 0x3380, 0x3380], dtype=np.uint16)
    rows4 = [np.tile(np.array([col[i], col[3 - i]], dtype=np.uint16), 5000) for i in range(4)]
    cb4, ocb4 = codebooks(rows4)
    R4, t4 = check_reduce_k(rows4, 256, cb4, ocb4, "order k=4")
    y4 = host_words(uzip.decode(R4, cb4, rows4[0].size, 256, in_bytes=t4))
    assert y4[0] == 0x3F80 and y4[1] == 0x3F81


def test_reduce_k_shards_small():
    w = workloads.reduce_shards(8, buckets=4, bucket=1 << 14)
    cb, ocb = codebooks(list(w.x))
    check_reduce_k(list(w.x), 1024, cb, ocb, "shards small k=8")


@pytest.mark.timeout(900)
def test_reduce_k_shards_full():
    w = workloads.reduce_shards(8)
    rows = list(w.x)
    print(f"{w.name}: inputs ready", flush=True)
    ocb = oracle.calibrate(*rows)
    hist = None
    for r in rows:
        hist = uzip.histogram(to_dev(r), hist)
    cb = uzip.codebook_from_hist(hist.cpu().numpy().astype(np.uint64))
    assert list(cb.dec) == ocb.dec.tolist()
    check_reduce_k(rows, 1024, cb, ocb, "shards full k=8 x 2^26")


@pytest.mark.parametrize("k", [3, 2])
def test_tiles_with_more_escapes_than_the_lds_list(k):
    """Sums that mostly miss the codebook: a tile with more output escapes
    than the kernel's LDS escape list holds (6,144 of a tile's 8,192 words)
    lists them straight into its staging slot. The stream must still equal
    the oracle's byte for byte."""
    n, C = 50_003, 1024
    rng = np.random.default_rng(4242 + k)
    rows = [rng.integers(0, 1 << 16, n, dtype=np.uint16) for _ in range(k)]
    # a codebook of exponents the sums of uniform words almost never take:
    # the 16 smallest (a sum lands there only if every input is that small,
    # or by cancellation)
    hist = np.zeros(256, dtype=np.uint64)
    hist[0:16] = np.arange(16, 0, -1, dtype=np.uint64)
    cb = uzip.codebook_from_hist(hist)
    ocb = oracle.top16(hist)
    R, tr = check_reduce_k(rows, C, cb, ocb, f"k={k} overflowing tiles")
    # the stream (equal to the oracle's) has tiles over the LDS list's capacity
    secs = oracle.sections(R[:tr].cpu().numpy())
    offs = secs["offsets"].astype(np.int64)
    tile_chunks = 8192 // C
    per_tile = [offs[min(t + tile_chunks, secs["nchunks"])] - offs[t] for t in range(0, secs["nchunks"], tile_chunks)]
    assert max(per_tile) > 6144, per_tile
