"""Lossless split-exponent BF16 codec for AMD MI355X (gfx950).

The codec and its kernels live in the HIP library ``libuzip.so`` (C-ABI in
``include/uzip.h``); :mod:`lossless_bf16_tensor_amd.uzip` is a thin ctypes
binding over it that takes torch tensors for device memory and streams.
"""
from . import uzip  # noqa: F401
from .uzip import (Codebook, UzipError, calibrate, codebook_from_hist, decode,  # noqa: F401
                   encode, histogram, max_bytes, reduce_add, stream_bytes, validate,
                   validate_host, workspace_bytes)
