"""Seeded synthetic BF16 inputs for the split-exponent codec.

This module only draws numbers. It holds none of the codec's arithmetic: no
exponent split, no codebook, no rounding of sums. Values are drawn in float64
with NumPy's PCG64 ``default_rng(seed)``, cast to float32, and turned into
BF16 bit patterns with torch's CPU float32 -> bfloat16 conversion
(round-to-nearest-even), a library routine.

The shapes and value distributions stand in for the KV activations the
SplitZip page measures on ("SplitZip: Ultra Fast Lossless KV Compression for
Disaggregated LLM Serving", section 4.1: a 256M-value BF16 workload of
Qwen3-32B KV tensors, chunk size 1024). Those tensors need trained weights and
a dataset; these recipes draw values of the same shape and similar spread
instead. Every recipe draws in the order written below, so a seed fixes the
tensor bit for bit for a given NumPy version.

Each ``config_k`` returns a ``Workload``:
    x       uint16 array (or a tuple of two for the reduce workload)
    calib   uint16 array(s) whose exponent histogram builds the codebook
    chunks  chunk sizes C to encode with
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload", "bf16_bits", "config_1", "config_2", "config_3", "config_4",
    "config_5", "config", "reduce_shards", "kv_cache_e5m2", "e5m2_bits", "all_patterns", "random_words", "CONFIG_NAMES",
]

CONFIG_NAMES = {
    1: "tiny-codec-check-1M",
    2: "kv-layer-tile-16384x8x128",
    3: "kv-cache-2x64x2048x8x128",
    4: "escape-stress-t2.5-64M",
    5: "grad-reduce-2x512M",
}


@dataclasses.dataclass
class Workload:
    name: str
    x: object            # np.ndarray[uint16] or tuple of two
    calib: object        # np.ndarray[uint16] or tuple of arrays
    chunks: tuple
    shape: tuple
    recipe: str


def bf16_bits(f) -> np.ndarray:
    """float64/float32 array -> uint16 BF16 bit patterns (torch CPU RNE cast)."""
    import torch
    f32 = np.ascontiguousarray(np.asarray(f, dtype=np.float32)).reshape(-1)
    out = np.empty(f32.size, dtype=np.uint16)
    step = 1 << 24
    for s in range(0, f32.size, step):
        t = torch.from_numpy(f32[s:s + step]).to(torch.bfloat16)
        out[s:s + step] = t.view(torch.int16).numpy().view(np.uint16)
    return out


def e5m2_bits(f) -> np.ndarray:
    """float64/float32 array -> uint8 FP8 E5M2 bit patterns (torch CPU cast,
    round to nearest even)."""
    import torch
    f32 = np.ascontiguousarray(np.asarray(f, dtype=np.float32)).reshape(-1)
    out = np.empty(f32.size, dtype=np.uint8)
    step = 1 << 24
    for s in range(0, f32.size, step):
        t = torch.from_numpy(f32[s:s + step]).to(torch.float8_e5m2)
        out[s:s + step] = t.view(torch.uint8).numpy()
    return out


def _spiky_normal(seed: int, n: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n)
    k = int(round(0.005 * n))
    idx = rng.choice(n, k, replace=False)
    sgn = rng.integers(0, 2, k) * 2 - 1
    p = rng.integers(-60, 61, k)
    x[idx] = sgn * np.power(2.0, p.astype(np.float64))
    return bf16_bits(x)


def config_1(n: int = 1 << 20, seed: int = 0, calib_seed: int = 1,
             calib_n: int = 65536) -> Workload:
    """N(0,1) with 0.5 % of entries replaced by +-2^k, k uniform in [-60, 60]."""
    x = _spiky_normal(seed, n)
    cal = _spiky_normal(calib_seed, calib_n)
    return Workload(CONFIG_NAMES[1], x, cal, (1024,), (n,),
                    f"normal+0.5% spikes, seed {seed}; calib seed {calib_seed} n={calib_n}")


def config_2(tokens: int = 16384, seed: int = 2, calib_tokens: int = 1024) -> Workload:
    """[tokens, 8, 128]: N(0,1) x per-(head, dim) LogNormal(0,1) scale; 0.1 % of
    tokens have all their values multiplied by 64."""
    rng = np.random.default_rng(seed)
    s = np.exp(rng.standard_normal((8, 128)))
    z = rng.standard_normal((tokens, 8, 128))
    x = z * s
    n_out = int(round(0.001 * tokens))
    out = rng.choice(tokens, n_out, replace=False)
    x[out] *= 64.0
    bits = bf16_bits(x)
    cal = bits[: calib_tokens * 8 * 128].copy()
    return Workload(CONFIG_NAMES[2], bits, cal, (1024,), (tokens, 8, 128),
                    f"seed {seed}; {n_out} outlier tokens x64; calib first {calib_tokens} tokens")


def _kv_cache(seed: int, layers: int, tokens: int, only_layer0: bool = False, cast=None):
    """KV cache [2, layers, tokens, 8, 128] drawn block by block, cast to BF16
    (or by `cast`, e.g. e5m2_bits).

    Draw order: per-layer scale, per-channel scale, K bias, then for kv in
    (K, V) and each layer a [tokens, 8, 128] block of N(0,1).
    """
    cast = cast or bf16_bits
    dt = np.uint8 if cast is e5m2_bits else np.uint16
    rng = np.random.default_rng(seed)
    sl = np.exp(rng.uniform(math.log(0.05), math.log(20.0), layers))
    ch = np.exp(0.8 * rng.standard_normal((2, layers, 8, 128)))
    b = rng.standard_normal((layers, 8, 128))
    blk = tokens * 8 * 128
    if only_layer0:
        out = np.empty(2 * blk, dtype=dt)
    else:
        out = np.empty(2 * layers * blk, dtype=dt)
    for kv in (0, 1):
        for l in range(layers):
            z = rng.standard_normal((tokens, 8, 128))
            if kv == 0:
                z += b[l]
            block = z * sl[l] * ch[kv, l]
            if only_layer0:
                if l == 0:
                    out[kv * blk:(kv + 1) * blk] = cast(block)
            else:
                o = (kv * layers + l) * blk
                out[o:o + blk] = cast(block)
    return out


def config_3(tokens: int = 2048, layers: int = 64, seed: int = 3,
             calib_seed: int = 103) -> Workload:
    """KV cache shaped like a 32B dense model, [2, 64, 2048, 8, 128] = 2^28.

    Per-layer scale log-uniform in [0.05, 20]; per-channel LogNormal(0, 0.8);
    V = z*s*c, K = (z + bias)*s*c with a N(0,1) bias per (layer, head, dim).
    The codebook comes from layer 0 (K and V) of the same recipe drawn wholly
    from another seed.
    """
    x = _kv_cache(seed, layers, tokens)
    cal = _kv_cache(calib_seed, layers, tokens, only_layer0=True)
    return Workload(CONFIG_NAMES[3], x, cal, (1024,), (2, layers, tokens, 8, 128),
                    f"seed {seed}; calib layer 0 of seed {calib_seed}")


def kv_cache_e5m2(tokens: int = 2048, layers: int = 64, seed: int = 3, calib_seed: int = 103) -> Workload:
    """Config 3's KV cache recipe cast to FP8 E5M2 (one byte per value), the
    FP8 variant's workload; the codebook again from layer 0 of another seed."""
    x = _kv_cache(seed, layers, tokens, cast=e5m2_bits)
    cal = _kv_cache(calib_seed, layers, tokens, only_layer0=True, cast=e5m2_bits)
    return Workload(f"kv-cache-e5m2-2x{layers}x{tokens}x8x128", x, cal, (1024,), (2, layers, tokens, 8, 128),
                    f"seed {seed}; calib layer 0 of seed {calib_seed}; FP8 E5M2")


def config_4(n: int = 1 << 26, seed: int = 4, block: int = 4096,
             draw: int = 1 << 22) -> Workload:
    """Student-t (nu = 2.5) times 10^U(-4, 2), one scale per 4096-value block.
    The codebook is calibrated on the input itself."""
    rng = np.random.default_rng(seed)
    sc = 10.0 ** rng.uniform(-4.0, 2.0, n // block)
    out = np.empty(n, dtype=np.uint16)
    per = draw // block
    for i in range(n // draw):
        t = rng.standard_t(2.5, draw)
        v = t * np.repeat(sc[i * per:(i + 1) * per], block)
        out[i * draw:(i + 1) * draw] = bf16_bits(v)
    return Workload(CONFIG_NAMES[4], out, out, (256, 1024, 4096), (n,),
                    f"seed {seed}; t(2.5) x 10^U(-4,2) per {block}")


def _grad_buffer(seed: int, buckets: int, bucket: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    sig = np.exp(rng.uniform(math.log(1e-5), math.log(1e-2), buckets))
    out = np.empty(buckets * bucket, dtype=np.uint16)
    for bi in range(buckets):
        out[bi * bucket:(bi + 1) * bucket] = bf16_bits(sig[bi] * rng.standard_normal(bucket))
    return out


def config_5(buckets: int = 512, bucket: int = 1 << 20, seed_a: int = 50,
             seed_b: int = 51) -> Workload:
    """Two gradient buffers, N(0, sigma) with sigma log-uniform in [1e-5, 1e-2]
    per 2^20-value bucket, each buffer from its own seed. The codebook comes
    from the two buffers' exponent histograms added together."""
    a = _grad_buffer(seed_a, buckets, bucket)
    b = _grad_buffer(seed_b, buckets, bucket)
    return Workload(CONFIG_NAMES[5], (a, b), (a, b), (1024,), (buckets * bucket,),
                    f"seeds {seed_a}/{seed_b}; {buckets} buckets of {bucket}")


def reduce_shards(k: int = 8, buckets: int = 64, bucket: int = 1 << 20, seed0: int = 60) -> Workload:
    """One GPU's share of the gradient-reduce step done as a two-shot
    all-reduce over k GPUs: the shard of each GPU's buffer that this GPU
    reduces. Each of the k shards follows the gradient-buffer recipe of
    config 5 (sigma log-uniform in [1e-5, 1e-2] per 2^20-value bucket) with
    its own seed, seed0 + i; at the default size a shard is 2^26 values, the
    eighth of a config-5 buffer. The codebook comes from the k shards'
    histograms added together."""
    xs = tuple(_grad_buffer(seed0 + i, buckets, bucket) for i in range(k))
    return Workload(f"reduce-shards-{k}x{buckets * bucket}", xs, xs, (1024,), (buckets * bucket,),
                    f"seeds {seed0}..{seed0 + k - 1}; {buckets} buckets of {bucket} per shard")


def config(k: int, small: bool = False) -> Workload:
    """Config k at its stated size, or (small=True) the same recipe at a size
    the oracle handles in about a second."""
    if k == 1:
        return config_1()
    if k == 2:
        return config_2(tokens=1024 + 512 if small else 16384)
    if k == 3:
        return config_3(tokens=8, layers=8) if small else config_3()
    if k == 4:
        return config_4(n=1 << 21, draw=1 << 19) if small else config_4()
    if k == 5:
        return config_5(buckets=8, bucket=1 << 16) if small else config_5()
    raise ValueError(f"no config {k}")


def all_patterns(seed: int = 0) -> np.ndarray:
    """Every 16-bit word exactly once, in a seeded random order."""
    rng = np.random.default_rng(seed)
    return rng.permutation(65536).astype(np.uint16)


def random_words(n: int, seed: int) -> np.ndarray:
    """n uniformly random 16-bit words."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 65536, n, dtype=np.uint16)
