"""ctypes binding of libuzip.so (C-ABI: include/uzip.h).

Argument marshalling only: every step of the codec runs in the library's HIP
kernels. torch supplies device memory (tensors) and the stream
(``torch.cuda.current_stream()``). The library must be built first
(``python -m lossless_bf16_tensor_amd.build``); without it every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# UZIP_LIB points the binding at another build of the same library (the CPU
# sanitizer test loads a host-instrumented build this way).
LIB_PATH = os.environ.get("UZIP_LIB", os.path.join(_HERE, "libuzip.so"))

UZIP_VERSION = 1
UZIP_F_SEPARATE_PATCH = 0x1
ERRORS = {0: "UZIP_OK", -1: "UZIP_EINVAL", -2: "UZIP_ENOSPC", -3: "UZIP_ECORRUPT",
          -4: "UZIP_ECODEBOOK", -5: "UZIP_EHIP", -6: "UZIP_ESCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20        # UZIP_NOALLOC_SCRATCH_BYTES

# every symbol include/uzip.h declares
EXPORTS = (
    "uzip_max_bytes", "uzip_workspace_bytes", "uzip_codebook_from_hist", "uzip_codebook_from_dec",
    "uzip_validate_host", "uzip_parse_header", "uzip_strerror", "uzip_histogram", "uzip_histogram_sampled",
    "uzip_calibrate", "uzip_encode", "uzip_encode_ex", "uzip_encode_online", "uzip_encode_online_ex",
    "uzip_stream_bytes", "uzip_decode", "uzip_decode_ex", "uzip_reduce_add", "uzip_reduce_add_ex",
    "uzip_reduce_k", "uzip_reduce_k_ex", "uzip_validate", "uzip_fp8_max_bytes", "uzip_fp8_histogram",
    "uzip_fp8_calibrate", "uzip_fp8_encode", "uzip_fp8_encode_ex", "uzip_fp8_decode", "uzip_fp8_decode_ex",
    "uzip_s15_max_bytes", "uzip_s15_encode", "uzip_s15_encode_ex", "uzip_s15_decode", "uzip_s15_decode_ex",
    "uzip_z7_max_bytes", "uzip_z7_encode", "uzip_z7_encode_ex", "uzip_z7_decode", "uzip_z7_decode_ex",
    "uzip_t8_max_bytes", "uzip_t8_encode", "uzip_t8_encode_ex", "uzip_t8_decode", "uzip_t8_decode_ex",
    "uzip_encode_noalloc",
)

MAX_K = 16                      # UZIP_MAX_K


class UzipError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class Codebook(ctypes.Structure):
    """uzip_codebook_t: dec[16], enc[256], member[256], hist[256], n_cal."""
    _fields_ = [("version", ctypes.c_uint32), ("dec", ctypes.c_uint8 * 16),
                ("enc", ctypes.c_uint8 * 256), ("member", ctypes.c_uint8 * 256),
                ("hist", ctypes.c_uint64 * 256), ("n_cal", ctypes.c_uint64)]

    @property
    def dec_list(self):
        return list(self.dec)


class Opts(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("n_events", ctypes.c_uint32),
                ("flags", ctypes.c_uint32)]


_lib = None


def lib():
    """Load libuzip.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m lossless_bf16_tensor_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, u64, u32, i32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
    cbp = ctypes.POINTER(Codebook)
    op = ctypes.POINTER(Opts)
    sig = {
        "uzip_max_bytes": (u64, [u64, u32]),
        "uzip_workspace_bytes": (u64, [u64, u32]),
        "uzip_codebook_from_hist": (i32, [vp, cbp]),
        "uzip_codebook_from_dec": (i32, [vp, cbp]),
        "uzip_validate_host": (i32, [vp, u64, cbp]),
        "uzip_parse_header": (i32, [vp, vp, vp, vp, vp, vp]),
        "uzip_strerror": (ctypes.c_char_p, [i32]),
        "uzip_histogram": (i32, [vp, u64, vp, vp]),
        "uzip_histogram_sampled": (i32, [vp, u64, u64, u64, vp, vp]),
        "uzip_calibrate": (i32, [vp, u64, vp, cbp, vp]),
        "uzip_encode": (i32, [vp, u64, u32, cbp, vp, u64, vp, u64, vp]),
        "uzip_encode_ex": (i32, [vp, u64, u32, cbp, vp, u64, vp, u64, op, vp]),
        "uzip_encode_noalloc": (i32, [vp, u64, u32, cbp, vp, u64, vp]),
        "uzip_encode_online": (i32, [vp, u64, u32, u64, u64, vp, vp, u64, vp, u64, vp]),
        "uzip_encode_online_ex": (i32, [vp, u64, u32, u64, u64, vp, vp, u64, vp, u64, op, vp]),
        "uzip_stream_bytes": (i32, [vp, vp, vp, vp]),
        "uzip_decode": (i32, [vp, u64, u64, u32, cbp, vp, vp]),
        "uzip_decode_ex": (i32, [vp, u64, u64, u32, cbp, vp, op, vp]),
        "uzip_reduce_add": (i32, [vp, u64, vp, u64, u64, u32, cbp, vp, u64, vp, u64, vp]),
        "uzip_reduce_add_ex": (i32, [vp, u64, vp, u64, u64, u32, cbp, vp, u64, vp, u64, op, vp]),
        "uzip_reduce_k": (i32, [ctypes.POINTER(vp), ctypes.POINTER(u64), u32, u64, u32, cbp, vp, u64, vp, u64,
                                vp]),
        "uzip_reduce_k_ex": (i32, [ctypes.POINTER(vp), ctypes.POINTER(u64), u32, u64, u32, cbp, vp, u64, vp,
                                   u64, op, vp]),
        "uzip_validate": (i32, [vp, u64, cbp, vp]),
        "uzip_s15_max_bytes": (u64, [u64, u32]),
        "uzip_s15_encode": (i32, [vp, u64, u32, cbp, vp, u64, vp, u64, vp]),
        "uzip_s15_encode_ex": (i32, [vp, u64, u32, cbp, vp, u64, vp, u64, op, vp]),
        "uzip_s15_decode": (i32, [vp, u64, u64, u32, cbp, vp, vp]),
        "uzip_s15_decode_ex": (i32, [vp, u64, u64, u32, cbp, vp, op, vp]),
        "uzip_t8_max_bytes": (u64, [u64, u32]),
        "uzip_t8_encode": (i32, [vp, u64, u32, cbp, vp, u64, vp, u64, vp]),
        "uzip_t8_encode_ex": (i32, [vp, u64, u32, cbp, vp, u64, vp, u64, op, vp]),
        "uzip_t8_decode": (i32, [vp, u64, u64, u32, cbp, vp, vp]),
        "uzip_t8_decode_ex": (i32, [vp, u64, u64, u32, cbp, vp, op, vp]),
        "uzip_z7_max_bytes": (u64, [u64, u32]),
        "uzip_z7_encode": (i32, [vp, u64, u32, cbp, vp, u64, vp, u64, vp]),
        "uzip_z7_encode_ex": (i32, [vp, u64, u32, cbp, vp, u64, vp, u64, op, vp]),
        "uzip_z7_decode": (i32, [vp, u64, u64, u32, cbp, vp, vp]),
        "uzip_z7_decode_ex": (i32, [vp, u64, u64, u32, cbp, vp, op, vp]),
        "uzip_fp8_max_bytes": (u64, [u64, u32]),
        "uzip_fp8_histogram": (i32, [vp, u64, vp, vp]),
        "uzip_fp8_calibrate": (i32, [vp, u64, vp, cbp, vp]),
        "uzip_fp8_encode": (i32, [vp, u64, u32, cbp, vp, u64, vp, u64, vp]),
        "uzip_fp8_encode_ex": (i32, [vp, u64, u32, cbp, vp, u64, vp, u64, op, vp]),
        "uzip_fp8_decode": (i32, [vp, u64, u64, u32, cbp, vp, vp]),
        "uzip_fp8_decode_ex": (i32, [vp, u64, u64, u32, cbp, vp, op, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(rc: int, what: str):
    if rc != 0:
        raise UzipError(rc, f"{what}: {lib().uzip_strerror(rc).decode()}")


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _empty(n, dtype, device, stream=None, zero=False):
    """A new device tensor that belongs to `stream` (None: the current
    stream). The caching allocator hands a freed block only to later work on
    the stream the block belongs to, so a temporary that a call's kernels use
    on `stream` cannot be reused by other streams' work while they run."""
    if stream is None:
        return torch.zeros(n, dtype=dtype, device=device) if zero else torch.empty(n, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.zeros(n, dtype=dtype, device=device) if zero else torch.empty(n, dtype=dtype, device=device)


def _ptr(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _words(t: torch.Tensor) -> torch.Tensor:
    """View a bfloat16/int16/uint16 tensor as flat 16-bit words."""
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    if t.dtype not in (torch.int16, torch.uint16):
        raise ValueError(f"expected 16-bit words, got {t.dtype}")
    return t.reshape(-1)


def _opts(events=None, flags=0):
    if not events and not flags:
        return None
    o = Opts()
    if events:
        arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
        o.events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        o.n_events = len(events)
        o._keep = arr
    o.flags = flags
    return o


# ------------------------------------------------------------- host only ----
def max_bytes(n: int, chunk: int) -> int:
    return int(lib().uzip_max_bytes(n, chunk))


def workspace_bytes(n: int, chunk: int) -> int:
    return int(lib().uzip_workspace_bytes(n, chunk))


def codebook_from_hist(hist) -> Codebook:
    h = (ctypes.c_uint64 * 256)(*[int(v) for v in hist])
    cb = Codebook()
    _check(lib().uzip_codebook_from_hist(ctypes.cast(h, ctypes.c_void_p), ctypes.byref(cb)),
           "codebook_from_hist")
    return cb


def codebook_from_dec(dec) -> Codebook:
    """The codebook with decode table dec[16] (hist and n_cal zero)."""
    d = (ctypes.c_uint8 * 16)(*[int(v) for v in dec])
    cb = Codebook()
    _check(lib().uzip_codebook_from_dec(ctypes.cast(d, ctypes.c_void_p), ctypes.byref(cb)), "codebook_from_dec")
    return cb


def validate_host(buf: bytes, cb: Codebook) -> int:
    """Structural check of a host copy of a stream; returns the C status code."""
    b = bytes(buf)
    return int(lib().uzip_validate_host(ctypes.c_char_p(b), len(b), ctypes.byref(cb)))


def parse_header(buf: bytes):
    b = bytes(buf[:256])
    n, m, tot = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    c = ctypes.c_uint32()
    dec = (ctypes.c_uint8 * 16)()
    _check(lib().uzip_parse_header(ctypes.c_char_p(b), ctypes.byref(n), ctypes.byref(c),
                                   ctypes.byref(m), ctypes.byref(tot), ctypes.cast(dec, ctypes.c_void_p)),
           "parse_header")
    return {"n": n.value, "chunk": c.value, "m": m.value, "total_bytes": tot.value, "dec": list(dec)}


# ---------------------------------------------------------------- device ----
def histogram(x: torch.Tensor, hist: torch.Tensor | None = None, block: int = 0, sample: int = 0,
              stream=None) -> torch.Tensor:
    """Add the exponent histogram of x to hist (int64[256] on the device).
    With block > 0, only the first `sample` words of every `block` words
    are counted."""
    w = _words(x)
    if hist is None:
        hist = _empty(256, torch.int64, w.device, stream, zero=True)
    if block:
        _check(lib().uzip_histogram_sampled(_ptr(w), w.numel(), block, sample, _ptr(hist), _stream(stream)),
               "histogram_sampled")
    else:
        _check(lib().uzip_histogram(_ptr(w), w.numel(), _ptr(hist), _stream(stream)), "histogram")
    return hist


def calibrate(x: torch.Tensor, stream=None) -> Codebook:
    w = _words(x)
    ws = _empty(256, torch.int64, w.device, stream)
    cb = Codebook()
    _check(lib().uzip_calibrate(_ptr(w), w.numel(), _ptr(ws), ctypes.byref(cb), _stream(stream)),
           "calibrate")
    return cb


def encode(x: torch.Tensor, cb: Codebook, chunk: int = 1024, out: torch.Tensor | None = None,
           ws: torch.Tensor | None = None, events=None, stream=None) -> torch.Tensor:
    """Encode; returns the uint8 output buffer (max_bytes long). The stream's
    own size is in its header (stream_bytes)."""
    w = _words(x)
    n = w.numel()
    cap = max_bytes(n, chunk)
    if cap == 0:
        raise UzipError(-1, f"bad n={n} or chunk={chunk}")
    if out is None:
        out = _empty(cap, torch.uint8, w.device, stream)
    if ws is None:
        ws = _empty(workspace_bytes(n, chunk), torch.uint8, w.device, stream)
    o = _opts(events)
    _check(lib().uzip_encode_ex(_ptr(w), n, chunk, ctypes.byref(cb), _ptr(out), out.numel(),
                                _ptr(ws), ws.numel(), ctypes.byref(o) if o else None, _stream(stream)),
           "encode")
    return out


def encode_noalloc(x: torch.Tensor, cb: Codebook, chunk: int = 1024, out: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """encode() through uzip_encode_noalloc: the library allocates nothing
    and uses its fixed per-GPU scratch as the workspace (calls on one GPU
    must not overlap). With out given, this allocates nothing either."""
    w = _words(x)
    n = w.numel()
    if out is None:
        out = _empty(max_bytes(n, chunk), torch.uint8, w.device, stream)
    _check(lib().uzip_encode_noalloc(_ptr(w), n, chunk, ctypes.byref(cb), _ptr(out), out.numel(), _stream(stream)),
           "encode_noalloc")
    return out


def encode_online(x: torch.Tensor, chunk: int = 1024, block: int = 0, sample: int = 0,
                  out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                  cb_out: torch.Tensor | None = None, events=None, stream=None) -> torch.Tensor:
    """Encode with a codebook calibrated on x on the device (block = 0: the
    whole of x; else the first `sample` words of every `block` words).
    cb_out, if given, is a uint8 device tensor of ctypes.sizeof(Codebook)
    bytes that receives the codebook."""
    w = _words(x)
    n = w.numel()
    if out is None:
        out = _empty(max_bytes(n, chunk), torch.uint8, w.device, stream)
    if ws is None:
        ws = _empty(workspace_bytes(n, chunk), torch.uint8, w.device, stream)
    if cb_out is not None and cb_out.numel() < ctypes.sizeof(Codebook):
        raise ValueError("cb_out is smaller than a codebook")
    o = _opts(events)
    _check(lib().uzip_encode_online_ex(_ptr(w), n, chunk, block, sample,
                                       _ptr(cb_out) if cb_out is not None else None, _ptr(out), out.numel(),
                                       _ptr(ws), ws.numel(), ctypes.byref(o) if o else None, _stream(stream)),
           "encode_online")
    return out


def codebook_of_device(cb_out: torch.Tensor) -> Codebook:
    """Host copy of a codebook that encode_online wrote to a device buffer."""
    b = bytes(cb_out[:ctypes.sizeof(Codebook)].cpu().numpy().tobytes())
    return Codebook.from_buffer_copy(b)


def stream_bytes(buf: torch.Tensor, stream=None):
    """(total_bytes, M) from a device stream's header (blocking)."""
    tot, m = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().uzip_stream_bytes(_ptr(buf), ctypes.byref(tot), ctypes.byref(m), _stream(stream)),
           "stream_bytes")
    return tot.value, m.value


def decode(buf: torch.Tensor, cb: Codebook, n: int, chunk: int = 1024, out: torch.Tensor | None = None,
           in_bytes: int | None = None, separate_patch: bool = False, events=None,
           stream=None) -> torch.Tensor:
    """Decode n words; returns an int16 tensor of BF16 bit patterns."""
    if out is None:
        out = _empty(n, torch.int16, buf.device, stream)
    w = _words(out)
    o = _opts(events, UZIP_F_SEPARATE_PATCH if separate_patch else 0)
    nb = buf.numel() if in_bytes is None else in_bytes
    _check(lib().uzip_decode_ex(_ptr(buf), nb, n, chunk, ctypes.byref(cb), _ptr(w),
                                ctypes.byref(o) if o else None, _stream(stream)), "decode")
    return out


def reduce_add(a: torch.Tensor, b: torch.Tensor, cb: Codebook, n: int, chunk: int = 1024,
               out: torch.Tensor | None = None, ws: torch.Tensor | None = None, events=None,
               stream=None) -> torch.Tensor:
    """Fused decode(a) + decode(b) -> binary32 add -> BF16 (RNE) -> encode."""
    cap = max_bytes(n, chunk)
    if out is None:
        out = _empty(cap, torch.uint8, a.device, stream)
    if ws is None:
        ws = _empty(workspace_bytes(n, chunk), torch.uint8, a.device, stream)
    o = _opts(events)
    _check(lib().uzip_reduce_add_ex(_ptr(a), a.numel(), _ptr(b), b.numel(), n, chunk, ctypes.byref(cb),
                                    _ptr(out), out.numel(), _ptr(ws), ws.numel(),
                                    ctypes.byref(o) if o else None, _stream(stream)), "reduce_add")
    return out


def reduce_k(streams, cb: Codebook, n: int, chunk: int = 1024, out: torch.Tensor | None = None,
             ws: torch.Tensor | None = None, events=None, stream=None) -> torch.Tensor:
    """Fused k-input reduce of uint8 device streams (each tensor's numel bounds
    its reads): decode all, add in binary32 in list order, round once to BF16,
    encode."""
    k = len(streams)
    if out is None:
        out = _empty(max_bytes(n, chunk), torch.uint8, streams[0].device, stream)
    if ws is None:
        ws = _empty(workspace_bytes(n, chunk), torch.uint8, streams[0].device, stream)
    ptrs = (ctypes.c_void_p * max(k, 1))(*[_ptr(t) for t in streams])
    sizes = (ctypes.c_uint64 * max(k, 1))(*[t.numel() for t in streams])
    o = _opts(events)
    _check(lib().uzip_reduce_k_ex(ptrs, sizes, k, n, chunk, ctypes.byref(cb), _ptr(out), out.numel(),
                                  _ptr(ws), ws.numel(), ctypes.byref(o) if o else None, _stream(stream)),
           "reduce_k")
    return out


def validate(buf: torch.Tensor, cb: Codebook, nbytes: int | None = None, stream=None) -> int:
    """Full structural check of a device stream (blocking); returns the status code."""
    if nbytes is None:
        nbytes, _ = stream_bytes(buf, stream)
    return int(lib().uzip_validate(_ptr(buf), nbytes, ctypes.byref(cb), _stream(stream)))


# ------------------------------------------------------------ FP8 E5M2 ----
def _bytes(t: torch.Tensor) -> torch.Tensor:
    """View a float8_e5m2/uint8/int8 tensor as flat bytes."""
    if t.dtype == torch.float8_e5m2:
        t = t.view(torch.uint8)
    if t.dtype not in (torch.uint8, torch.int8):
        raise ValueError(f"expected 8-bit values, got {t.dtype}")
    return t.reshape(-1)


def fp8_max_bytes(n: int, chunk: int) -> int:
    return int(lib().uzip_fp8_max_bytes(n, chunk))


def fp8_histogram(x: torch.Tensor, hist: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    b = _bytes(x)
    if hist is None:
        hist = _empty(256, torch.int64, b.device, stream, zero=True)
    _check(lib().uzip_fp8_histogram(_ptr(b), b.numel(), _ptr(hist), _stream(stream)), "fp8_histogram")
    return hist


def fp8_calibrate(x: torch.Tensor, stream=None) -> Codebook:
    b = _bytes(x)
    ws = _empty(256, torch.int64, b.device, stream)
    cb = Codebook()
    _check(lib().uzip_fp8_calibrate(_ptr(b), b.numel(), _ptr(ws), ctypes.byref(cb), _stream(stream)),
           "fp8_calibrate")
    return cb


def fp8_encode(x: torch.Tensor, cb: Codebook, chunk: int = 1024, out: torch.Tensor | None = None,
               ws: torch.Tensor | None = None, events=None, stream=None) -> torch.Tensor:
    b = _bytes(x)
    n = b.numel()
    if out is None:
        out = _empty(fp8_max_bytes(n, chunk), torch.uint8, b.device, stream)
    if ws is None:
        ws = _empty(workspace_bytes(n, chunk), torch.uint8, b.device, stream)
    o = _opts(events)
    _check(lib().uzip_fp8_encode_ex(_ptr(b), n, chunk, ctypes.byref(cb), _ptr(out), out.numel(), _ptr(ws),
                                    ws.numel(), ctypes.byref(o) if o else None, _stream(stream)), "fp8_encode")
    return out


def fp8_decode(buf: torch.Tensor, cb: Codebook, n: int, chunk: int = 1024, out: torch.Tensor | None = None,
               in_bytes: int | None = None, events=None, stream=None) -> torch.Tensor:
    """Decode n E5M2 values; returns a uint8 tensor."""
    if out is None:
        out = _empty(n, torch.uint8, buf.device, stream)
    o = _opts(events)
    nb = buf.numel() if in_bytes is None else in_bytes
    _check(lib().uzip_fp8_decode_ex(_ptr(buf), nb, n, chunk, ctypes.byref(cb), _ptr(out),
                                    ctypes.byref(o) if o else None, _stream(stream)), "fp8_decode")
    return out


# --------------------------------------------- Top-15 + sentinel --------
def s15_max_bytes(n: int, chunk: int) -> int:
    return int(lib().uzip_s15_max_bytes(n, chunk))


def s15_encode(x: torch.Tensor, cb: Codebook, chunk: int = 1024, out: torch.Tensor | None = None,
               ws: torch.Tensor | None = None, events=None, stream=None) -> torch.Tensor:
    w = _words(x)
    n = w.numel()
    if out is None:
        out = _empty(s15_max_bytes(n, chunk), torch.uint8, w.device, stream)
    if ws is None:
        ws = _empty(workspace_bytes(n, chunk), torch.uint8, w.device, stream)
    o = _opts(events)
    _check(lib().uzip_s15_encode_ex(_ptr(w), n, chunk, ctypes.byref(cb), _ptr(out), out.numel(), _ptr(ws),
                                    ws.numel(), ctypes.byref(o) if o else None, _stream(stream)), "s15_encode")
    return out


def s15_decode(buf: torch.Tensor, cb: Codebook, n: int, chunk: int = 1024, out: torch.Tensor | None = None,
               in_bytes: int | None = None, events=None, stream=None) -> torch.Tensor:
    if out is None:
        out = _empty(n, torch.int16, buf.device, stream)
    w = _words(out)
    o = _opts(events)
    nb = buf.numel() if in_bytes is None else in_bytes
    _check(lib().uzip_s15_decode_ex(_ptr(buf), nb, n, chunk, ctypes.byref(cb), _ptr(w),
                                    ctypes.byref(o) if o else None, _stream(stream)), "s15_decode")
    return out


# ------------------------------------ Top-7 3-bit + zero-point ----------
def z7_max_bytes(n: int, chunk: int) -> int:
    return int(lib().uzip_z7_max_bytes(n, chunk))


def z7_encode(x: torch.Tensor, cb: Codebook, chunk: int = 1024, out: torch.Tensor | None = None,
              ws: torch.Tensor | None = None, events=None, stream=None) -> torch.Tensor:
    w = _words(x)
    n = w.numel()
    if out is None:
        out = _empty(z7_max_bytes(n, chunk), torch.uint8, w.device, stream)
    if ws is None:
        ws = _empty(workspace_bytes(n, chunk), torch.uint8, w.device, stream)
    o = _opts(events)
    _check(lib().uzip_z7_encode_ex(_ptr(w), n, chunk, ctypes.byref(cb), _ptr(out), out.numel(), _ptr(ws),
                                   ws.numel(), ctypes.byref(o) if o else None, _stream(stream)), "z7_encode")
    return out


def z7_decode(buf: torch.Tensor, cb: Codebook, n: int, chunk: int = 1024, out: torch.Tensor | None = None,
              in_bytes: int | None = None, events=None, stream=None) -> torch.Tensor:
    if out is None:
        out = _empty(n, torch.int16, buf.device, stream)
    w = _words(out)
    o = _opts(events)
    nb = buf.numel() if in_bytes is None else in_bytes
    _check(lib().uzip_z7_decode_ex(_ptr(buf), nb, n, chunk, ctypes.byref(cb), _ptr(w),
                                   ctypes.byref(o) if o else None, _stream(stream)), "z7_decode")
    return out


# --------------------------------------- Top-8 3-bit with positions -----
def t8_max_bytes(n: int, chunk: int) -> int:
    return int(lib().uzip_t8_max_bytes(n, chunk))


def t8_encode(x: torch.Tensor, cb: Codebook, chunk: int = 1024, out: torch.Tensor | None = None,
              ws: torch.Tensor | None = None, events=None, stream=None) -> torch.Tensor:
    w = _words(x)
    n = w.numel()
    if out is None:
        out = _empty(t8_max_bytes(n, chunk), torch.uint8, w.device, stream)
    if ws is None:
        ws = _empty(workspace_bytes(n, chunk), torch.uint8, w.device, stream)
    o = _opts(events)
    _check(lib().uzip_t8_encode_ex(_ptr(w), n, chunk, ctypes.byref(cb), _ptr(out), out.numel(), _ptr(ws),
                                   ws.numel(), ctypes.byref(o) if o else None, _stream(stream)), "t8_encode")
    return out


def t8_decode(buf: torch.Tensor, cb: Codebook, n: int, chunk: int = 1024, out: torch.Tensor | None = None,
              in_bytes: int | None = None, events=None, stream=None) -> torch.Tensor:
    if out is None:
        out = _empty(n, torch.int16, buf.device, stream)
    w = _words(out)
    o = _opts(events)
    nb = buf.numel() if in_bytes is None else in_bytes
    _check(lib().uzip_t8_decode_ex(_ptr(buf), nb, n, chunk, ctypes.byref(cb), _ptr(w),
                                   ctypes.byref(o) if o else None, _stream(stream)), "t8_decode")
    return out
