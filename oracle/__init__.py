"""CPU oracle for the split-exponent lossless BF16 codec (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product (the HIP library and its
Python binding) never imports it.

The arithmetic lives in ``uzip_oracle.c`` (plain scalar C, built with gcc);
this module only marshals NumPy arrays through ctypes. See that file's header
for the passages each function follows and the readings taken where the pages
leave a point open.

Parity status: split/merge, histogram, Top-16, encode, decode, the reduce's
rounding, the k-input reduce's summation order, and the FP8, Top-15 +
sentinel, Top-7 3-bit + zero-point and Top-8 3-bit formats are pinned by the tests under
``tests/test_oracle_*.py``. The one
choice the pages do not fix at all -- a NaN sum in the reduce becomes 0x7FC0 --
is "parity unpinned" (it is our own convention).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "uzip_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test that plants a mistake in a copy of the oracle points this at the copy.
_LIB = os.environ.get("UZIP_ORACLE_LIB", _LIB)

_lib = None


def build(sanitize: bool = False, out: str | None = None) -> str:
    """Compile the oracle with gcc (IEEE binary32, no fast-math, no FMA).
    sanitize=True adds AddressSanitizer and UndefinedBehaviorSanitizer (a
    process loading that build must preload gcc's libasan)."""
    lib = out or _LIB
    san = (["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
           if sanitize else [])
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-msse2", "-mfpmath=sse", "-Wall", "-Wextra", *san,
           "-o", lib + ".tmp", _SRC]
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if "UZIP_ORACLE_LIB" not in os.environ and (
            not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        build()
    L = ctypes.CDLL(_LIB)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    c64, c32 = ctypes.c_uint64, ctypes.c_uint32
    sig = {
        "orc_exponent": (ctypes.c_uint8, [ctypes.c_uint16]),
        "orc_signmant": (ctypes.c_uint8, [ctypes.c_uint16]),
        "orc_merge": (ctypes.c_uint16, [ctypes.c_uint8, ctypes.c_uint8]),
        "orc_histogram": (None, [u16p, c64, u64p]),
        "orc_top16": (None, [u64p, u8p, u8p, u8p]),
        "orc_max_bytes": (c64, [c64, c32]),
        "orc_payload_bytes": (c64, [c64, c64]),
        "orc_encode": (c64, [u16p, c64, c32, u8p, u8p, c64]),
        "orc_decode": (ctypes.c_int, [u8p, c64, c64, c32, u8p, u16p]),
        "orc_bf16_rne": (ctypes.c_uint16, [c32]),
        "orc_add_bf16": (ctypes.c_uint16, [ctypes.c_uint16, ctypes.c_uint16]),
        "orc_reduce_add": (c64, [u8p, c64, u8p, c64, c64, c32, u8p, u8p, c64, u16p]),
        "orc_validate": (ctypes.c_int, [u8p, c64, u8p]),
        "orc_stream_m": (c64, [u8p]),
        "orc_stream_total": (c64, [u8p]),
        "orc_bf16_rne_array": (None, [ctypes.POINTER(ctypes.c_uint32), c64, u16p]),
        "orc_add_bf16_array": (None, [u16p, u16p, c64, u16p]),
        "orc_sum_bf16": (ctypes.c_uint16, [u16p, c32, c64]),
        "orct8_max_bytes": (c64, [c64, c32]),
        "orct8_payload_bytes": (c64, [c64, c64]),
        "orct8_encode": (c64, [u16p, c64, c32, u8p, u8p, c64]),
        "orct8_decode": (ctypes.c_int, [u8p, c64, c64, c32, u8p, u16p]),
        "orct8_validate": (ctypes.c_int, [u8p, c64, u8p]),
        "orcz_max_bytes": (c64, [c64, c32]),
        "orcz_payload_bytes": (c64, [c64, c64]),
        "orcz_encode": (c64, [u16p, c64, c32, u8p, u8p, c64]),
        "orcz_decode": (ctypes.c_int, [u8p, c64, c64, c32, u8p, u16p]),
        "orcz_validate": (ctypes.c_int, [u8p, c64, u8p]),
        "orcs_max_bytes": (c64, [c64, c32]),
        "orcs_payload_bytes": (c64, [c64, c64]),
        "orcs_encode": (c64, [u16p, c64, c32, u8p, u8p, c64]),
        "orcs_decode": (ctypes.c_int, [u8p, c64, c64, c32, u8p, u16p]),
        "orcs_validate": (ctypes.c_int, [u8p, c64, u8p]),
        "orc8_exponent": (ctypes.c_uint8, [ctypes.c_uint8]),
        "orc8_signmant": (ctypes.c_uint8, [ctypes.c_uint8]),
        "orc8_merge": (ctypes.c_uint8, [ctypes.c_uint8, ctypes.c_uint8]),
        "orc8_histogram": (None, [u8p, c64, u64p]),
        "orc8_max_bytes": (c64, [c64, c32]),
        "orc8_payload_bytes": (c64, [c64, c64]),
        "orc8_encode": (c64, [u8p, c64, c32, u8p, u8p, c64]),
        "orc8_decode": (ctypes.c_int, [u8p, c64, c64, c32, u8p, u8p]),
        "orc8_validate": (ctypes.c_int, [u8p, c64, u8p]),
        "orc_reduce_k": (c64, [ctypes.POINTER(u8p), u64p, c32, c64, c32, u8p, u8p, c64, u16p]),
        "orc_sum_bf16_array": (None, [u16p, c32, c64, u16p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _p(a, t):
    return a.ctypes.data_as(ctypes.POINTER(t))


def _u16(x):
    return np.ascontiguousarray(x, dtype=np.uint16)


# ------------------------------------------------------------------ scalars --
def exponent(x: int) -> int:
    return int(_load().orc_exponent(x))


def signmant(x: int) -> int:
    return int(_load().orc_signmant(x))


def merge(a: int, e: int) -> int:
    return int(_load().orc_merge(a, e))


def bf16_rne(u32: int) -> int:
    return int(_load().orc_bf16_rne(u32))


def add_bf16(a: int, b: int) -> int:
    return int(_load().orc_add_bf16(a, b))


# ---------------------------------------------------------------- codebook --
class Codebook:
    """dec[16] (code -> exponent), enc[256] (exponent -> code, 0 if absent),
    member[256] (1 if the exponent has a code), and the histogram it came from."""

    def __init__(self, dec, enc, member, hist):
        self.dec = np.asarray(dec, dtype=np.uint8)
        self.enc = np.asarray(enc, dtype=np.uint8)
        self.member = np.asarray(member, dtype=np.uint8)
        self.hist = np.asarray(hist, dtype=np.uint64)


def histogram(*arrays) -> np.ndarray:
    """Exponent histogram pooled over one or more uint16 arrays."""
    L = _load()
    h = np.zeros(256, dtype=np.uint64)
    for x in arrays:
        x = _u16(x)
        L.orc_histogram(_p(x, ctypes.c_uint16), x.size, _p(h, ctypes.c_uint64))
    return h


def top16(hist) -> Codebook:
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    dec = np.zeros(16, np.uint8)
    enc = np.zeros(256, np.uint8)
    mem = np.zeros(256, np.uint8)
    _load().orc_top16(_p(h, ctypes.c_uint64), _p(dec, ctypes.c_uint8),
                      _p(enc, ctypes.c_uint8), _p(mem, ctypes.c_uint8))
    return Codebook(dec, enc, mem, h)


def calibrate(*arrays) -> Codebook:
    return top16(histogram(*arrays))


# ------------------------------------------------------------------- codec --
def max_bytes(n: int, chunk: int) -> int:
    return int(_load().orc_max_bytes(n, chunk))


def payload_bytes(n: int, m: int) -> int:
    return int(_load().orc_payload_bytes(n, m))


def encode(x, chunk: int, dec) -> np.ndarray:
    """Encode uint16 words; returns the stream as a uint8 array."""
    x = _u16(x).reshape(-1)
    dec = np.ascontiguousarray(dec, dtype=np.uint8)
    cap = max_bytes(x.size, chunk)
    out = np.empty(cap, dtype=np.uint8)
    total = _load().orc_encode(_p(x, ctypes.c_uint16), x.size, chunk,
                               _p(dec, ctypes.c_uint8), _p(out, ctypes.c_uint8), cap)
    if total == 0:
        raise ValueError("oracle encode rejected its arguments")
    return out[:total].copy()


def decode(stream, n: int, chunk: int, dec) -> np.ndarray:
    s = np.ascontiguousarray(stream, dtype=np.uint8)
    dec = np.ascontiguousarray(dec, dtype=np.uint8)
    y = np.empty(n, dtype=np.uint16)
    rc = _load().orc_decode(_p(s, ctypes.c_uint8), s.size, n, chunk,
                            _p(dec, ctypes.c_uint8), _p(y, ctypes.c_uint16))
    if rc != 0:
        raise ValueError("oracle decode: stream does not match its arguments")
    return y


def reduce_add(sa, sb, n: int, chunk: int, dec) -> np.ndarray:
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    dec = np.ascontiguousarray(dec, dtype=np.uint8)
    cap = max_bytes(n, chunk)
    out = np.empty(cap, dtype=np.uint8)
    tmp = np.empty(3 * n, dtype=np.uint16)
    total = _load().orc_reduce_add(_p(sa, ctypes.c_uint8), sa.size, _p(sb, ctypes.c_uint8), sb.size,
                                   n, chunk, _p(dec, ctypes.c_uint8), _p(out, ctypes.c_uint8), cap,
                                   _p(tmp, ctypes.c_uint16))
    if total == 0:
        raise ValueError("oracle reduce_add failed")
    return out[:total].copy()


def sample_words(x, block: int, sample: int) -> np.ndarray:
    """The calibration sample of x: the first `sample` words of every block
    of `block` words, the last block possibly partial ("CCCL", section 4.3,
    localized frequency tables: a table from the first part of each block's
    range). block = 0 means all of x."""
    x = _u16(x).reshape(-1)
    if block == 0:
        return x.copy()
    parts = [x[b:b + sample] for b in range(0, x.size, block)]
    return np.concatenate(parts) if parts else x[:0].copy()


def reduce_k(streams, n: int, chunk: int, dec) -> np.ndarray:
    """k-input reduce of compressed streams (same n, chunk and codebook)."""
    arrs = [np.ascontiguousarray(x, dtype=np.uint8) for x in streams]
    k = len(arrs)
    dec = np.ascontiguousarray(dec, dtype=np.uint8)
    cap = max_bytes(n, chunk)
    out = np.empty(cap, dtype=np.uint8)
    tmp = np.empty((k + 1) * n, dtype=np.uint16)
    ptrs = (ctypes.POINTER(ctypes.c_uint8) * max(k, 1))(*[_p(x, ctypes.c_uint8) for x in arrs])
    sizes = (ctypes.c_uint64 * max(k, 1))(*[x.size for x in arrs])
    total = _load().orc_reduce_k(ptrs, sizes, k, n, chunk, _p(dec, ctypes.c_uint8),
                                 _p(out, ctypes.c_uint8), cap, _p(tmp, ctypes.c_uint16))
    if total == 0:
        raise ValueError("oracle reduce_k failed")
    return out[:total].copy()


def sum_words(rows) -> np.ndarray:
    """k-input reduce arithmetic on raw words (no codec): rows is (k, n)."""
    v = np.ascontiguousarray(rows, dtype=np.uint16)
    if v.ndim != 2:
        raise ValueError("rows must be (k, n)")
    k, n = v.shape
    r = np.empty(n, dtype=np.uint16)
    _load().orc_sum_bf16_array(_p(v, ctypes.c_uint16), k, n, _p(r, ctypes.c_uint16))
    return r


def add_words(a, b) -> np.ndarray:
    """Element-wise reduce arithmetic on raw words (no codec)."""
    a = _u16(a).reshape(-1)
    b = _u16(b).reshape(-1)
    r = np.empty(a.size, dtype=np.uint16)
    _load().orc_add_bf16_array(_p(a, ctypes.c_uint16), _p(b, ctypes.c_uint16), a.size,
                               _p(r, ctypes.c_uint16))
    return r


def bf16_rne_words(u32) -> np.ndarray:
    """binary32 bit patterns -> BF16 words, the reduce's final rounding."""
    u = np.ascontiguousarray(u32, dtype=np.uint32).reshape(-1)
    r = np.empty(u.size, dtype=np.uint16)
    _load().orc_bf16_rne_array(_p(u, ctypes.c_uint32), u.size, _p(r, ctypes.c_uint16))
    return r


def validate(stream, dec) -> int:
    s = np.ascontiguousarray(stream, dtype=np.uint8)
    dec = np.ascontiguousarray(dec, dtype=np.uint8)
    return int(_load().orc_validate(_p(s, ctypes.c_uint8), s.size, _p(dec, ctypes.c_uint8)))


def stream_m(stream) -> int:
    s = np.ascontiguousarray(stream, dtype=np.uint8)
    return int(_load().orc_stream_m(_p(s, ctypes.c_uint8)))


# ----------------------------------------------------------- section views --
def sections(stream) -> dict:
    """Split a stream into its sections (reads the header's n, C, M)."""
    s = np.asarray(stream, dtype=np.uint8)
    n = int(s[16:24].view(np.uint64)[0])
    C = int(s[8:12].view(np.uint32)[0])
    m = int(s[24:32].view(np.uint64)[0])
    A = lambda v: (v + 255) & ~255
    nch = (n + C - 1) // C
    sm = 256
    codes = sm + A(n)
    offs = codes + A((n + 1) // 2)
    pos = offs + A(4 * (nch + 1))
    val = pos + A(2 * m)
    return {
        "n": n, "C": C, "m": m, "nchunks": nch,
        "sm": s[sm:sm + n], "codes": s[codes:codes + (n + 1) // 2],
        "offsets": s[offs:offs + 4 * (nch + 1)].view(np.uint32),
        "pos": s[pos:pos + 2 * m].view(np.uint16), "val": s[val:val + m],
        "dec": s[40:56].copy(), "total": int(s[32:40].view(np.uint64)[0]),
    }


# ----------------------------------------------------------- FP8 E5M2 ----
def _u8(x):
    return np.ascontiguousarray(x, dtype=np.uint8)


def fp8_exponent(x: int) -> int:
    return int(_load().orc8_exponent(x))


def fp8_signmant(x: int) -> int:
    return int(_load().orc8_signmant(x))


def fp8_merge(a: int, e: int) -> int:
    return int(_load().orc8_merge(a, e))


def fp8_histogram(*sets) -> np.ndarray:
    """Pooled 256-bin histogram of the 5-bit exponents of E5M2 values."""
    hist = np.zeros(256, dtype=np.uint64)
    for x in sets:
        x = _u8(x).reshape(-1)
        _load().orc8_histogram(_p(x, ctypes.c_uint8), x.size, _p(hist, ctypes.c_uint64))
    return hist


def fp8_calibrate(*sets) -> Codebook:
    return top16(fp8_histogram(*sets))


def fp8_max_bytes(n: int, chunk: int) -> int:
    return int(_load().orc8_max_bytes(n, chunk))


def fp8_payload_bytes(n: int, m: int) -> int:
    return int(_load().orc8_payload_bytes(n, m))


def fp8_encode(x, chunk: int, dec) -> np.ndarray:
    x = _u8(x).reshape(-1)
    dec = _u8(dec)
    cap = fp8_max_bytes(x.size, chunk)
    out = np.empty(cap, dtype=np.uint8)
    total = _load().orc8_encode(_p(x, ctypes.c_uint8), x.size, chunk, _p(dec, ctypes.c_uint8),
                                _p(out, ctypes.c_uint8), cap)
    if total == 0:
        raise ValueError("oracle fp8 encode failed")
    return out[:total].copy()


def fp8_decode(stream, n: int, chunk: int, dec) -> np.ndarray:
    stream = _u8(stream)
    dec = _u8(dec)
    y = np.empty(n, dtype=np.uint8)
    rc = _load().orc8_decode(_p(stream, ctypes.c_uint8), stream.size, n, chunk, _p(dec, ctypes.c_uint8),
                             _p(y, ctypes.c_uint8))
    if rc != 0:
        raise ValueError("oracle fp8 decode failed")
    return y


def fp8_validate(stream, dec) -> int:
    stream = _u8(stream)
    dec = _u8(dec)
    return int(_load().orc8_validate(_p(stream, ctypes.c_uint8), stream.size, _p(dec, ctypes.c_uint8)))


# ------------------------------------------------ Top-15 + sentinel ----
def s15_max_bytes(n: int, chunk: int) -> int:
    return int(_load().orcs_max_bytes(n, chunk))


def s15_payload_bytes(n: int, m: int) -> int:
    return int(_load().orcs_payload_bytes(n, m))


def s15_encode(x, chunk: int, dec) -> np.ndarray:
    x = _u16(x).reshape(-1)
    dec = _u8(dec)
    cap = s15_max_bytes(x.size, chunk)
    out = np.empty(cap, dtype=np.uint8)
    total = _load().orcs_encode(_p(x, ctypes.c_uint16), x.size, chunk, _p(dec, ctypes.c_uint8),
                                _p(out, ctypes.c_uint8), cap)
    if total == 0:
        raise ValueError("oracle s15 encode failed")
    return out[:total].copy()


def s15_decode(stream, n: int, chunk: int, dec) -> np.ndarray:
    stream = _u8(stream)
    dec = _u8(dec)
    y = np.empty(n, dtype=np.uint16)
    rc = _load().orcs_decode(_p(stream, ctypes.c_uint8), stream.size, n, chunk, _p(dec, ctypes.c_uint8),
                             _p(y, ctypes.c_uint16))
    if rc != 0:
        raise ValueError("oracle s15 decode failed")
    return y


def s15_validate(stream, dec) -> int:
    stream = _u8(stream)
    dec = _u8(dec)
    return int(_load().orcs_validate(_p(stream, ctypes.c_uint8), stream.size, _p(dec, ctypes.c_uint8)))


# --------------------------------------- Top-7 3-bit + zero-point ------
def z7_max_bytes(n: int, chunk: int) -> int:
    return int(_load().orcz_max_bytes(n, chunk))


def z7_payload_bytes(n: int, m: int) -> int:
    return int(_load().orcz_payload_bytes(n, m))


def z7_encode(x, chunk: int, dec) -> np.ndarray:
    x = _u16(x).reshape(-1)
    dec = _u8(dec)
    cap = z7_max_bytes(x.size, chunk)
    out = np.empty(cap, dtype=np.uint8)
    total = _load().orcz_encode(_p(x, ctypes.c_uint16), x.size, chunk, _p(dec, ctypes.c_uint8),
                                _p(out, ctypes.c_uint8), cap)
    if total == 0:
        raise ValueError("oracle z7 encode failed")
    return out[:total].copy()


def z7_decode(stream, n: int, chunk: int, dec) -> np.ndarray:
    stream = _u8(stream)
    dec = _u8(dec)
    y = np.empty(n, dtype=np.uint16)
    rc = _load().orcz_decode(_p(stream, ctypes.c_uint8), stream.size, n, chunk, _p(dec, ctypes.c_uint8),
                             _p(y, ctypes.c_uint16))
    if rc != 0:
        raise ValueError("oracle z7 decode failed")
    return y


def z7_validate(stream, dec) -> int:
    stream = _u8(stream)
    dec = _u8(dec)
    return int(_load().orcz_validate(_p(stream, ctypes.c_uint8), stream.size, _p(dec, ctypes.c_uint8)))


# ---------------------------------------- Top-8 3-bit with positions ----
def t8_max_bytes(n: int, chunk: int) -> int:
    return int(_load().orct8_max_bytes(n, chunk))


def t8_payload_bytes(n: int, m: int) -> int:
    return int(_load().orct8_payload_bytes(n, m))


def t8_encode(x, chunk: int, dec) -> np.ndarray:
    x = _u16(x).reshape(-1)
    dec = _u8(dec)
    cap = t8_max_bytes(x.size, chunk)
    out = np.empty(cap, dtype=np.uint8)
    total = _load().orct8_encode(_p(x, ctypes.c_uint16), x.size, chunk, _p(dec, ctypes.c_uint8),
                                 _p(out, ctypes.c_uint8), cap)
    if total == 0:
        raise ValueError("oracle t8 encode failed")
    return out[:total].copy()


def t8_decode(stream, n: int, chunk: int, dec) -> np.ndarray:
    stream = _u8(stream)
    dec = _u8(dec)
    y = np.empty(n, dtype=np.uint16)
    rc = _load().orct8_decode(_p(stream, ctypes.c_uint8), stream.size, n, chunk, _p(dec, ctypes.c_uint8),
                              _p(y, ctypes.c_uint16))
    if rc != 0:
        raise ValueError("oracle t8 decode failed")
    return y


def t8_validate(stream, dec) -> int:
    stream = _u8(stream)
    dec = _u8(dec)
    return int(_load().orct8_validate(_p(stream, ctypes.c_uint8), stream.size, _p(dec, ctypes.c_uint8)))
