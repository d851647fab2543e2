"""Chunk-parallel driver around the unchanged CPU oracle (test infrastructure).

Only ``tests/`` and the CPU-baseline leg of ``bench.py`` use it. It adds no
arithmetic of the codec: the input is cut at chunk boundaries into one piece
per thread, each piece is encoded (or decoded) by the oracle's own
``orc_encode`` / ``orc_decode`` in its own thread (ctypes releases the GIL
for the call), and the pieces are put together by the stream layout alone:
the dense sections and the escape arrays concatenated in piece order, each
piece's chunk offsets shifted by the escapes of the pieces before it (a
serial prefix over the pieces), and the header's n, M and total size set.

Chunks are independent except for that prefix (the escape arrays of the
SplitZip review, section 3.2, are per chunk), so the joined stream equals
the one-thread stream byte for byte; ``tests/test_cpu_parallel.py`` checks
that on every shape it runs.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

from . import decode, encode, histogram, reduce_add, sections


def _a256(v: int) -> int:
    return (v + 255) & ~255


def default_threads(cap: int = 16) -> int:
    """The cores this process may run on (at most `cap`)."""
    return max(1, min(cap, len(os.sched_getaffinity(0))))


def piece_bounds(n: int, chunk: int, parts: int):
    """[(c0, c1)] chunk ranges, one per piece, in order (no empty piece)."""
    nch = (n + chunk - 1) // chunk
    parts = max(1, min(parts, nch))
    per = (nch + parts - 1) // parts
    return [(c, min(c + per, nch)) for c in range(0, nch, per)]


def join(pieces, n: int, chunk: int) -> np.ndarray:
    """One stream from the streams of consecutive chunk ranges of an input."""
    secs = [sections(p) for p in pieces]
    m = sum(s["m"] for s in secs)
    nch = (n + chunk - 1) // chunk
    off_codes = 256 + _a256(n)
    off_offs = off_codes + _a256((n + 1) // 2)
    off_pos = off_offs + _a256(4 * (nch + 1))
    off_val = off_pos + _a256(2 * m)
    total = off_val + m
    out = np.zeros(total, dtype=np.uint8)
    out[:256] = pieces[0][:256]
    out[16:24] = np.frombuffer(np.uint64(n).tobytes(), np.uint8)
    out[24:32] = np.frombuffer(np.uint64(m).tobytes(), np.uint8)
    out[32:40] = np.frombuffer(np.uint64(total).tobytes(), np.uint8)
    offs = out[off_offs:off_offs + 4 * (nch + 1)].view(np.uint32)
    pos = out[off_pos:off_pos + 2 * m].view(np.uint16)
    e0 = c0 = j0 = 0
    for s in secs:
        k, pc, pm = s["n"], s["nchunks"], s["m"]
        out[256 + e0:256 + e0 + k] = s["sm"]
        cb = e0 // 2                      # pieces other than the last hold whole chunks: e0 is even
        out[off_codes + cb:off_codes + cb + s["codes"].size] = s["codes"]
        offs[c0:c0 + pc] = s["offsets"][:pc] + np.uint32(j0)
        pos[j0:j0 + pm] = s["pos"]
        out[off_val + j0:off_val + j0 + pm] = s["val"]
        e0, c0, j0 = e0 + k, c0 + pc, j0 + pm
    offs[nch] = m
    return out


def split(stream, c0: int, c1: int) -> np.ndarray:
    """The stream of chunks [c0, c1) of a stream, as that piece's encode
    would write it."""
    s = sections(stream)
    n, C = s["n"], s["C"]
    e0, e1 = c0 * C, min(c1 * C, n)
    k = e1 - e0
    offs = s["offsets"]
    j0, j1 = int(offs[c0]), int(offs[c1])
    pm, pc = j1 - j0, c1 - c0
    off_codes = 256 + _a256(k)
    off_offs = off_codes + _a256((k + 1) // 2)
    off_pos = off_offs + _a256(4 * (pc + 1))
    off_val = off_pos + _a256(2 * pm)
    total = off_val + pm
    out = np.zeros(total, dtype=np.uint8)
    out[:256] = np.asarray(stream[:256], dtype=np.uint8)
    out[16:24] = np.frombuffer(np.uint64(k).tobytes(), np.uint8)
    out[24:32] = np.frombuffer(np.uint64(pm).tobytes(), np.uint8)
    out[32:40] = np.frombuffer(np.uint64(total).tobytes(), np.uint8)
    out[256:256 + k] = s["sm"][e0:e1]
    out[off_codes:off_codes + (k + 1) // 2] = s["codes"][e0 // 2:e0 // 2 + (k + 1) // 2]
    out[off_offs:off_offs + 4 * (pc + 1)].view(np.uint32)[:] = offs[c0:c1 + 1] - np.uint32(j0)
    out[off_pos:off_pos + 2 * pm].view(np.uint16)[:] = s["pos"][j0:j1]
    out[off_val:off_val + pm] = s["val"][j0:j1]
    return out


def encode_parallel(x, chunk: int, dec, threads: int | None = None, pool=None) -> np.ndarray:
    """oracle.encode(x, chunk, dec), with the chunks shared out over threads."""
    x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1)
    n = x.size
    bounds = piece_bounds(n, chunk, threads or default_threads())

    def one(b):
        return encode(x[b[0] * chunk:min(b[1] * chunk, n)], chunk, dec)

    if pool is None:
        with cf.ThreadPoolExecutor(len(bounds)) as p:
            pieces = list(p.map(one, bounds))
    else:
        pieces = list(pool.map(one, bounds))
    return join(pieces, n, chunk)


def decode_parallel(stream, n: int, chunk: int, dec, threads: int | None = None, pool=None) -> np.ndarray:
    """oracle.decode(stream, n, chunk, dec), with the chunks shared out over
    threads (each thread cuts its piece's stream out, then decodes it)."""
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    y = np.empty(n, dtype=np.uint16)
    bounds = piece_bounds(n, chunk, threads or default_threads())

    def one(b):
        e0, e1 = b[0] * chunk, min(b[1] * chunk, n)
        y[e0:e1] = decode(split(stream, *b), e1 - e0, chunk, dec)

    if pool is None:
        with cf.ThreadPoolExecutor(len(bounds)) as p:
            list(p.map(one, bounds))
    else:
        list(pool.map(one, bounds))
    return y


def reduce_add_parallel(sa, sb, n: int, chunk: int, dec, threads: int | None = None, pool=None) -> np.ndarray:
    """oracle.reduce_add(sa, sb, n, chunk, dec), with the chunks shared out
    over threads: each thread cuts the same chunk range out of both streams
    and reduces that pair of pieces; the results are joined."""
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    bounds = piece_bounds(n, chunk, threads or default_threads())

    def one(b):
        e0, e1 = b[0] * chunk, min(b[1] * chunk, n)
        return reduce_add(split(sa, *b), split(sb, *b), e1 - e0, chunk, dec)

    if pool is None:
        with cf.ThreadPoolExecutor(len(bounds)) as p:
            pieces = list(p.map(one, bounds))
    else:
        pieces = list(pool.map(one, bounds))
    return join(pieces, n, chunk)


def histogram_parallel(x, threads: int | None = None, pool=None) -> np.ndarray:
    """oracle.histogram(x), with x cut into one piece per thread: the pieces'
    histograms are counted by the oracle and added."""
    x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1)
    parts = max(1, min(threads or default_threads(), x.size))
    step = (x.size + parts - 1) // parts
    pieces = [x[i:i + step] for i in range(0, x.size, step)] or [x]
    if pool is None:
        with cf.ThreadPoolExecutor(len(pieces)) as p:
            hists = list(p.map(histogram, pieces))
    else:
        hists = list(pool.map(histogram, pieces))
    return np.sum(hists, axis=0, dtype=np.uint64)

