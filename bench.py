#!/usr/bin/env python3
"""Benchmark of the split-exponent BF16 codec on one MI355X.

Workload: the 2^28-value KV cache [K/V 2, layers 64, tokens 2048, kv_heads 8,
head_dim 128], drawn by the seeded recipe in workloads.config_3 (per-layer
log-uniform scale, per-channel log-normal scale, K bias). The codebook is
calibrated on layer 0 of the same recipe drawn from another seed. Chunk 1024.

A step is one round trip of the whole tensor: encode (dense pass, tile scan,
escape placement), then decode (fused dense decode + sparse patch). The input
and every buffer are resident in HBM before timing starts. Calibration runs
once, offline, before the timed region: the SplitZip page (section 3.3) moves
it out of the online path. Its time is reported separately, as is the fused
decode-add-reencode reduce on two such tensors.

Before timing, the GPU stream is compared byte for byte with the CPU oracle's,
and the round trip is checked bit for bit.

Output: one JSON line on stdout. value = uncompressed BF16 bytes (2N) per
second of a round-trip step, in GB/s (1e9). Per-op rates, the compression
ratio, the escape rate, the per-kernel HIP-event durations and the roofline of
the dominant kernel are extra fields.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(n, C, m):
    """Bytes the method must move (uncompressed in/out, compressed sections)."""
    nch = (n + C - 1) // C
    comp = n + (n + 1) // 2 + 3 * m + 4 * (nch + 1) + 256
    return {
        "encode": 2 * n + comp,                 # read words, write stream
        "decode": comp + 2 * n,                 # read stream, write words
        # dense pass: read words, write sign-mantissa and code sections
        "k_encode_tile": 2 * n + n + (n + 1) // 2,
        "k_decode_tile": comp + 2 * n,
    }


def stream_bytes_alg(n, C, m):
    """Algorithmic bytes of one compressed stream: the payload N + N/2 + 3M
    plus the chunk offsets and the header."""
    nch = (n + C - 1) // C
    return n + (n + 1) // 2 + 3 * m + 4 * (nch + 1) + 256


def stats_ms(vals):
    v = np.asarray(vals, dtype=np.float64)
    return {"mean": round(float(v.mean()), 4), "median": round(float(np.median(v)), 4),
            "min": round(float(v.min()), 4)}


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (two rocprofv3 --pmc passes, FETCH_SIZE and WRITE_SIZE, each scaled by a
    plain copy of known size), or None when the kernel source has changed
    since the counters were taken."""
    import glob
    import hashlib
    src = os.path.join(ROOT, "lossless_bf16_tensor_amd", "csrc", "uzip.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    for path in glob.glob(os.path.join(ROOT, "profiles", "*_hbm_counters.md")):
        text = open(path).read()
        if f"kernel_source_sha256_prefix: {sha}" not in text:
            continue
        for line in text.splitlines():
            if line.startswith(f"traffic_bytes {kernel}:"):
                return int(line.split(":")[1])
    return None


def entropy_bits(hist):
    p = hist[hist > 0].astype(np.float64) / hist.sum()
    return float(-(p * np.log2(p)).sum())


def cpu_baseline(x_np, calib_np, C, budget_s=12.0, sample=1 << 24):
    """The CPU oracle (plain C, untuned) on a bounded sample of the workload:
    once on one thread, then with the sample's chunks shared out over every
    core this process may use (oracle/parallel.py: the unchanged oracle per
    piece, a serial offsets prefix). The two streams must be identical."""
    import concurrent.futures as cf

    import oracle
    from oracle import parallel
    xs = np.ascontiguousarray(x_np[:sample])
    n = xs.size
    cb = oracle.calibrate(calib_np)

    def timed(enc, dec):
        reps, t_enc, t_dec = 0, 0.0, 0.0
        t_start = time.perf_counter()
        while reps < 5 and (reps == 0 or time.perf_counter() - t_start < budget_s):
            t0 = time.perf_counter()
            s = enc()
            t1 = time.perf_counter()
            y = dec(s)
            t2 = time.perf_counter()
            assert np.array_equal(y, xs)
            t_enc += t1 - t0
            t_dec += t2 - t1
            reps += 1
        gb = 2 * n * reps / 1e9
        return s, reps, gb / t_enc, gb / t_dec, gb / (t_enc + t_dec)

    s1, r1, e1, d1, v1 = timed(lambda: oracle.encode(xs, C, cb.dec), lambda s: oracle.decode(s, n, C, cb.dec))
    threads = parallel.default_threads()
    with cf.ThreadPoolExecutor(threads) as pool:
        sp, rp, ep, dp, vp = timed(lambda: parallel.encode_parallel(xs, C, cb.dec, threads, pool),
                                   lambda s: parallel.decode_parallel(s, n, C, cb.dec, threads, pool))
    assert np.array_equal(sp, s1), "chunk-parallel oracle stream differs from the one-thread stream"
    t0 = time.perf_counter()
    oracle.histogram(xs)                                                 # calibration's first step, one thread
    hist_gbps = 2 * n / (time.perf_counter() - t0) / 1e9
    m = int(np.frombuffer(s1[24:32].tobytes(), dtype="<u8")[0])         # header: M, then total bytes
    total = int(np.frombuffer(s1[32:40].tobytes(), dtype="<u8")[0])
    return {
        "value": round(vp, 4), "unit": "GB/s",
        "cores": threads, "kind": "oracle",
        "sample": f"first {n} values of the same workload, {rp} round trips on {threads} threads "
                  f"(chunks shared out, the unchanged oracle per piece; encode {ep:.4f} GB/s, decode {dp:.4f} GB/s); "
                  f"one thread: {r1} round trips, encode {e1:.4f} GB/s, decode {d1:.4f} GB/s",
        "encode_GBps": round(ep, 4), "decode_GBps": round(dp, 4),
        "one_thread": {"value": round(v1, 4), "encode_GBps": round(e1, 4), "decode_GBps": round(d1, 4),
                       "histogram_GBps": round(hist_gbps, 4), "cores": 1},
        "streams_identical": True,
        "cpu": _cpu_model(), "host_cores": len(os.sched_getaffinity(0)), "numpy": np.__version__,
        "sample_sha256": hashlib.sha256(xs.tobytes()).hexdigest()[:16],
        "oracle_escape_rate": round(m / n, 6),
        "oracle_ratio_payload": round(2 * n / (n + (n + 1) // 2 + 3 * m), 4),
        "oracle_ratio_total": round(2 * n / total, 4),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def make_flush(torch, dev, mib):
    """A callable that reads `mib` MiB on the current stream (0: a no-op).
    Reads allocate in the Infinity Cache, so they evict earlier contents,
    and they leave only clean lines behind."""
    if mib <= 0:
        return lambda: None
    buf = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    return lambda: buf.sum()


def table(uzip, torch, reps=10, flush_mib=1024):
    """One JSON line per (config, chunk): encode/decode (and, for the
    gradient-reduce config, fused reduce) throughput, ratio, escape rate, and
    the CPU oracle on a bounded sample, on one thread and on every core.
    Every row is gated on a bit-exact round trip."""
    import concurrent.futures as cf

    import oracle
    import workloads
    from oracle import parallel as oparallel
    dev = torch.device("cuda:0")
    flush = make_flush(torch, dev, flush_mib)   # evicts the Infinity Cache before each timed call

    for k in (1, 2, 3, 4, 5):
        log(f"config {k}: generating")
        w = workloads.config(k)
        xs = w.x if isinstance(w.x, tuple) else (w.x,)
        cals = w.calib if isinstance(w.calib, tuple) else (w.calib,)
        hist = None
        for c in cals:
            hist = uzip.histogram(torch.from_numpy(c.view(np.int16)).to(dev), hist)
        cb = uzip.codebook_from_hist(hist.cpu().numpy().astype(np.uint64))
        x_np = xs[0]
        n = x_np.size
        x = torch.from_numpy(x_np.view(np.int16)).to(dev)
        for C in w.chunks:
            out = torch.empty(uzip.max_bytes(n, C), dtype=torch.uint8, device=dev)
            ws = torch.empty(uzip.workspace_bytes(n, C), dtype=torch.uint8, device=dev)
            y = torch.empty(n, dtype=torch.int16, device=dev)
            uzip.encode(x, cb, C, out=out, ws=ws)
            total, m = uzip.stream_bytes(out)
            uzip.decode(out, cb, n, C, out=y, in_bytes=total)
            torch.cuda.synchronize()
            if not torch.equal(y, x):
                log(f"CORRECTNESS FAILURE config {k} C={C}")
                sys.exit(1)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
            for row in ev:
                for e in row:
                    e.record()
            for _ in range(3):
                uzip.encode(x, cb, C, out=out, ws=ws)
                uzip.decode(out, cb, n, C, out=y, in_bytes=total)
            for r in range(reps):
                flush()
                ev[r][0].record()
                uzip.encode(x, cb, C, out=out, ws=ws)
                ev[r][1].record()
                flush()
                ev[r][2].record()
                uzip.decode(out, cb, n, C, out=y, in_bytes=total)
                ev[r][3].record()
            torch.cuda.synchronize()
            te = [ev[r][0].elapsed_time(ev[r][1]) for r in range(reps)]
            td = [ev[r][2].elapsed_time(ev[r][3]) for r in range(reps)]
            ab = algorithmic_bytes(n, C, m)
            row = {"config": k, "workload": w.name, "n": n, "chunk": C, "M": m, "escape_rate": round(m / n, 6),
                   "ratio_payload": round(2 * n / (n + (n + 1) // 2 + 3 * m), 4),
                   "ratio_total": round(2 * n / total, 4),
                   "encode_ms_mean": round(float(np.mean(te)), 4), "encode_ms_median": round(float(np.median(te)), 4),
                   "decode_ms_mean": round(float(np.mean(td)), 4), "decode_ms_median": round(float(np.median(td)), 4),
                   "encode_GBps": round(2 * n / (np.mean(te) * 1e-3) / 1e9, 1),
                   "decode_GBps": round(2 * n / (np.mean(td) * 1e-3) / 1e9, 1),
                   "encode_roofline": round(ab["encode"] / (np.mean(te) * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                   "decode_roofline": round(ab["decode"] / (np.mean(td) * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
            if len(xs) == 2:
                b = torch.from_numpy(xs[1].view(np.int16)).to(dev)
                outb = torch.empty_like(out)
                outr = torch.empty_like(out)
                uzip.encode(b, cb, C, out=outb, ws=ws)
                tb, _ = uzip.stream_bytes(outb)
                for _ in range(2):
                    uzip.reduce_add(out[:total], outb[:tb], cb, n, C, out=outr, ws=ws)
                rev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
                for rr in rev:
                    for e in rr:
                        e.record()
                for r in range(reps):
                    flush()
                    rev[r][0].record()
                    uzip.reduce_add(out[:total], outb[:tb], cb, n, C, out=outr, ws=ws)
                    rev[r][1].record()
                torch.cuda.synchronize()
                tr = [rev[r][0].elapsed_time(rev[r][1]) for r in range(reps)]
                trr, mr = uzip.stream_bytes(outr)
                red_bytes = (total + tb) + trr
                row.update({"reduce_ms_mean": round(float(np.mean(tr)), 4),
                            "reduce_GBps_uncompressed_in": round(2 * 2 * n / (np.mean(tr) * 1e-3) / 1e9, 1),
                            "reduce_stream_roofline": round(red_bytes / (np.mean(tr) * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                            "reduce_escape_rate": round(mr / n, 6)})
                del b, outb, outr
            # the CPU oracle on a bounded sample (one thread)
            sample = min(n, 1 << 22)
            xs_np = np.ascontiguousarray(x_np[:sample])
            ocb = oracle.top16(hist.cpu().numpy().astype(np.uint64))
            t0 = time.perf_counter()
            st = oracle.encode(xs_np, C, ocb.dec)
            t1 = time.perf_counter()
            oracle.decode(st, sample, C, ocb.dec)
            t2 = time.perf_counter()
            oracle.histogram(xs_np)
            t3 = time.perf_counter()
            row.update({"oracle_sample": sample, "oracle_encode_GBps": round(2 * sample / (t1 - t0) / 1e9, 4),
                        "oracle_decode_GBps": round(2 * sample / (t2 - t1) / 1e9, 4),
                        "oracle_histogram_GBps": round(2 * sample / (t3 - t2) / 1e9, 4), "oracle_cores": 1})
            # the same sample with its chunks shared out over every core this
            # process may use; the streams must equal the one-thread ones
            threads = oparallel.default_threads()
            with cf.ThreadPoolExecutor(threads) as pool:
                t0 = time.perf_counter()
                sp = oparallel.encode_parallel(xs_np, C, ocb.dec, threads, pool)
                t1 = time.perf_counter()
                yp = oparallel.decode_parallel(st, sample, C, ocb.dec, threads, pool)
                t2 = time.perf_counter()
                hp = oparallel.histogram_parallel(xs_np, threads, pool)
                t3 = time.perf_counter()
                assert np.array_equal(sp, st) and np.array_equal(yp, xs_np), "all-core oracle differs"
                assert np.array_equal(hp, oracle.histogram(xs_np)), "all-core oracle histogram differs"
                row.update({"oracle_allcore_encode_GBps": round(2 * sample / (t1 - t0) / 1e9, 4),
                            "oracle_allcore_decode_GBps": round(2 * sample / (t2 - t1) / 1e9, 4),
                            "oracle_allcore_histogram_GBps": round(2 * sample / (t3 - t2) / 1e9, 4),
                            "oracle_allcore_cores": threads})
                if len(xs) == 2:
                    # the oracle's fused reduce on the same sample of both inputs
                    stb = oracle.encode(np.ascontiguousarray(xs[1][:sample]), C, ocb.dec)
                    t4 = time.perf_counter()
                    r1 = oracle.reduce_add(st, stb, sample, C, ocb.dec)
                    t5 = time.perf_counter()
                    rp = oparallel.reduce_add_parallel(st, stb, sample, C, ocb.dec, threads, pool)
                    t6 = time.perf_counter()
                    assert np.array_equal(rp, r1), "all-core oracle reduce differs"
                    row["oracle_reduce_GBps_uncompressed_in"] = round(2 * 2 * sample / (t5 - t4) / 1e9, 4)
                    row["oracle_allcore_reduce_GBps_uncompressed_in"] = round(2 * 2 * sample / (t6 - t5) / 1e9, 4)
            print("TABLE " + json.dumps(row), flush=True)
            del out, ws, y
        del x
        torch.cuda.empty_cache()


def reduce_config5(uzip, torch, dev, flush, C, reps=10):
    """The fused reduce at its own configuration: two 2^29-value gradient
    buffers (seeded recipe), one codebook from both histograms, both encoded,
    then decode-add-RNE-reencode timed with events between its kernels."""
    import workloads
    log("reduce: generating two 2^29-value gradient buffers")
    w = workloads.config(5)
    xa = torch.from_numpy(w.x[0].view(np.int16)).to(dev)
    xb = torch.from_numpy(w.x[1].view(np.int16)).to(dev)
    n = xa.numel()
    hist = uzip.histogram(xb, uzip.histogram(xa))
    cb = uzip.codebook_from_hist(hist.cpu().numpy().astype(np.uint64))
    ws = torch.empty(uzip.workspace_bytes(n, C), dtype=torch.uint8, device=dev)
    sa = uzip.encode(xa, cb, C, ws=ws)
    sb = uzip.encode(xb, cb, C, ws=ws)
    ta, ma = uzip.stream_bytes(sa)
    tb, mb = uzip.stream_bytes(sb)
    del xa, xb
    outr = torch.empty(uzip.max_bytes(n, C), dtype=torch.uint8, device=dev)
    for _ in range(3):
        uzip.reduce_add(sa[:ta], sb[:tb], cb, n, C, out=outr, ws=ws)
    rev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    oev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for row in rev + oev:
        for e in row:
            e.record()
    for k in range(reps):                       # events between the kernels
        flush()
        uzip.reduce_add(sa[:ta], sb[:tb], cb, n, C, out=outr, ws=ws, events=rev[k])
    for k in range(reps):                       # events around the call only
        flush()
        oev[k][0].record()
        uzip.reduce_add(sa[:ta], sb[:tb], cb, n, C, out=outr, ws=ws)
        oev[k][1].record()
    torch.cuda.synchronize()
    op = [oev[k][0].elapsed_time(oev[k][1]) for k in range(reps)]
    kt = float(np.mean([rev[k][0].elapsed_time(rev[k][1]) for k in range(reps)]))
    kg = float(np.mean([rev[k][1].elapsed_time(rev[k][2]) for k in range(reps)]))
    kp = float(np.mean([rev[k][2].elapsed_time(rev[k][3]) for k in range(reps)]))
    tr, mr = uzip.stream_bytes(outr)
    alg = stream_bytes_alg(n, C, ma) + stream_bytes_alg(n, C, mb) + stream_bytes_alg(n, C, mr)
    t = float(np.mean(op))
    # the tile kernel's own bytes: both inputs' streams read, the result's
    # dense sections written (its escapes go through the staging slots)
    kbytes = stream_bytes_alg(n, C, ma) + stream_bytes_alg(n, C, mb) + n + (n + 1) // 2
    del sa, sb, outr, ws
    return {"workload": f"{w.name}: two BF16 gradient buffers of {n} values, codebook from both histograms",
            "n": n, "chunk": C, "ms": stats_ms(op),
            "GBps_uncompressed_in": round(2 * 2 * n / (t * 1e-3) / 1e9, 1),
            "algorithmic_bytes": alg, "op_frac": round(alg / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "kernels_ms": {"k_reduce_tile": round(kt, 4), "k_group_sums": round(kg, 4), "k_place_escapes": round(kp, 4)},
            "k_reduce_tile_frac": round(kbytes / (kt * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "escape_rate_inputs": [round(ma / n, 6), round(mb / n, 6)], "escape_rate_out": round(mr / n, 6),
            "stream_bytes": [ta, tb, tr]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--chunk", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-oracle-check", action="store_true")
    ap.add_argument("--no-reduce", action="store_true")
    ap.add_argument("--no-reduce-k", action="store_true")
    ap.add_argument("--no-online", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--small", action="store_true", help="reduced-size workload (smoke)")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="run one plain 1 GiB device copy first, to scale HBM byte counters")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="MiB read from a scratch buffer before every timed codec call to evict "
                         "the Infinity Cache (0: back-to-back calls)")
    ap.add_argument("--table", action="store_true",
                    help="measure every configuration (one TABLE line each) instead of the headline")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the codec shards by chunk with no cross-GPU exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from lossless_bf16_tensor_amd import uzip

    uzip.lib()                       # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    C = args.chunk
    if args.table:
        table(uzip, torch, flush_mib=args.flush_mib)
        return

    if args.pmc_calibration:
        # a plain copy kernel of known size: 2^29 16-bit words, 1 GiB read + 1 GiB write
        a_ = torch.ones(1 << 29, dtype=torch.int16, device=dev)
        b_ = torch.empty_like(a_)
        b_.copy_(a_)
        torch.cuda.synchronize()
        del a_, b_

    log("generating workload")
    w = workloads.config(3, small=args.small)
    x_np = w.x
    n = x_np.size
    log(f"workload {w.name}: n={n}")
    x = torch.from_numpy(x_np.view(np.int16)).to(dev)
    cal = torch.from_numpy(w.calib.view(np.int16)).to(dev)
    stream = torch.cuda.current_stream()

    # --- calibration (offline step; timed on its own) ---
    cb = uzip.calibrate(cal)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        cb = uzip.calibrate(cal)
    t_cal = (time.perf_counter() - t0) / 5
    hist = np.array(list(cb.hist), dtype=np.uint64)

    out = torch.empty(uzip.max_bytes(n, C), dtype=torch.uint8, device=dev)
    ws = torch.empty(uzip.workspace_bytes(n, C), dtype=torch.uint8, device=dev)
    y = torch.empty(n, dtype=torch.int16, device=dev)

    # --- correctness gate: oracle stream and bit-exact round trip ---
    uzip.encode(x, cb, C, out=out, ws=ws)
    total, m = uzip.stream_bytes(out)
    uzip.decode(out, cb, n, C, out=y, in_bytes=total)
    torch.cuda.synchronize()
    round_trip = bool(torch.equal(y, x))
    parity = None
    if not args.no_oracle_check:
        import oracle
        log("oracle check")
        ocb = oracle.calibrate(w.calib)
        assert list(cb.dec) == ocb.dec.tolist(), "codebook differs from the oracle"
        want = oracle.encode(x_np, C, ocb.dec)
        parity = bool(want.size == total and np.array_equal(out[:total].cpu().numpy(), want))
    if not round_trip or parity is False:
        log(f"CORRECTNESS FAILURE round_trip={round_trip} parity={parity}")
        sys.exit(1)

    # --- timed round trips (no events inside the timed region) ---
    # With --flush-mib F > 0, every codec call is preceded by a read of F MiB
    # from a scratch buffer (a sum), which evicts the 256 MB Infinity Cache,
    # so neither call finds the other's output in the cache. A read, not a
    # write: a write-based flush would leave the cache full of dirty lines
    # whose write-back lands in the next call's time. The flushes' own time
    # is measured in a separate loop and subtracted.
    flush = make_flush(torch, dev, args.flush_mib)

    def step(ev=None):
        flush()
        uzip.encode(x, cb, C, out=out, ws=ws, events=ev[:4] if ev else None)
        flush()
        uzip.decode(out, cb, n, C, out=y, in_bytes=total, events=ev[4:] if ev else None)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    wall_flush = 0.0
    if args.flush_mib > 0:
        for _ in range(2):
            flush()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(2 * args.steps):
            flush()
        torch.cuda.synchronize()
        wall_flush = time.perf_counter() - t0
    ms_step = (wall - wall_flush) / args.steps * 1e3

    # --- per-kernel durations: HIP events recorded between the kernels of
    # each call, on the stream they run on (a second pass of K steps) ---
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for row in evs:                  # torch creates the HIP event on first record
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()

    def avg(i, j):
        return float(np.mean([evs[k][i].elapsed_time(evs[k][j]) for k in range(args.steps)]))

    kern = {
        "k_encode_tile": avg(0, 1), "k_group_sums": avg(1, 2), "k_place_escapes": avg(2, 3),
        "k_decode_tile": avg(4, 5),
    }

    # --- whole-op durations: events around each call only (a third pass; the
    # events between an encode's kernels above add a few us to the call) ---
    oevs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for row in oevs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for k in range(args.steps):
        flush()
        oevs[k][0].record()
        uzip.encode(x, cb, C, out=out, ws=ws)
        oevs[k][1].record()
        flush()
        oevs[k][2].record()
        uzip.decode(out, cb, n, C, out=y, in_bytes=total)
        oevs[k][3].record()
    torch.cuda.synchronize()
    enc_list = [oevs[k][0].elapsed_time(oevs[k][1]) for k in range(args.steps)]
    dec_list = [oevs[k][2].elapsed_time(oevs[k][3]) for k in range(args.steps)]
    t_enc = float(np.mean(enc_list))
    t_dec = float(np.mean(dec_list))
    ab = algorithmic_bytes(n, C, m)

    # --- work a call leaves behind: lines it leaves dirty in the memory-side
    # cache are written back during the next operation, outside the call's
    # own time (the encode's staging, written with ordinary stores so that
    # the placement finds it in that cache). Measured as the extra time of a
    # cache-evicting read right after one call, against the same read after
    # another such read; the round-trip value above already includes it ---
    def left_behind(call, reps=10):
        if args.flush_mib <= 0:
            return 0.0
        t = {"clean": [], "after": []}
        for r in range(reps + 2):
            for what in ("clean", "after"):
                flush()
                call() if what == "after" else flush()
                ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ea.record()
                flush()
                eb.record()
                torch.cuda.synchronize()
                if r >= 2:
                    t[what].append(ea.elapsed_time(eb))
        return max(0.0, float(np.median(t["after"]) - np.median(t["clean"])))

    behind = {"encode": left_behind(lambda: uzip.encode(x, cb, C, out=out, ws=ws)),
              "decode": left_behind(lambda: uzip.decode(out, cb, n, C, out=y, in_bytes=total))}
    op_frac_full = {"encode": ab["encode"] / ((t_enc + behind["encode"]) * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                    "decode": ab["decode"] / ((t_dec + behind["decode"]) * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    # roofline per op: each op's whole-call fraction and its dominant
    # (longest) kernel's own fraction; the line's roofline is the slower op's
    op_frac = {"encode": ab["encode"] / (t_enc * 1e-3) / 1e9 / HBM_PEAK_GBPS,
               "decode": ab["decode"] / (t_dec * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    op_kernels = {"encode": ("k_encode_tile", "k_group_sums", "k_place_escapes"), "decode": ("k_decode_tile",)}
    roofline_ops = {}
    for op_name, ks in op_kernels.items():
        dk = max(ks, key=lambda k: kern[k])
        kb = ab.get(dk)
        roofline_ops[op_name] = {
            "op_ms": stats_ms(enc_list if op_name == "encode" else dec_list),
            "op_algorithmic_bytes": ab[op_name], "op_frac": round(op_frac[op_name], 4),
            "dominant_kernel": dk, "kernel_ms_mean": round(kern[dk], 4),
            "kernel_algorithmic_bytes": kb,
            "kernel_frac": round(kb / (kern[dk] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4) if kb else None,
            "kernels_ms": {k: round(kern[k], 4) for k in ks}}
    slow_op = min(op_frac, key=op_frac.get)
    dom = roofline_ops[slow_op]["dominant_kernel"]
    achieved = ab[dom] / (kern[dom] * 1e-3) / 1e9

    # --- a plain device copy of 1 GiB in the same run, for context: the
    # rate a read-and-write stream reaches on this machine ---
    cpy_a = torch.empty(1 << 29, dtype=torch.int16, device=dev)
    cpy_b = torch.empty_like(cpy_a)
    cpy_b.copy_(cpy_a)
    cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5)]
    for k in range(5):
        flush()
        cev[k][0].record()
        cpy_b.copy_(cpy_a)
        cev[k][1].record()
    torch.cuda.synchronize()
    t_cpy = [cev[k][0].elapsed_time(cev[k][1]) for k in range(5)]
    copy_gbps = 2 * cpy_a.numel() * 2 / (float(np.median(t_cpy)) * 1e-3) / 1e9
    del cpy_a, cpy_b
    enc_gbps = 2 * n / (t_enc * 1e-3) / 1e9
    dec_gbps = 2 * n / (t_dec * 1e-3) / 1e9
    rho_payload = 2 * n / (n + (n + 1) // 2 + 3 * m)
    rho_total = 2 * n / total
    value = 2 * n / (ms_step * 1e-3) / 1e9

    # --- fused reduce: the gradient-reduce configuration (two 2^29-value
    # buffers), and a high-escape pair (the headline tensor and the same
    # tensor with its K and V halves swapped) ---
    reduce = reduce_hi = None
    if not args.no_reduce:
        b = torch.roll(x, shifts=n // 2)
        outb = torch.empty_like(out)
        outr = torch.empty_like(out)
        uzip.encode(b, cb, C, out=outb, ws=ws)
        tb, _ = uzip.stream_bytes(outb)
        rev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(10)]
        for row in rev:
            for e in row:
                e.record()
        for k in range(3):
            uzip.reduce_add(out[:total], outb[:tb], cb, n, C, out=outr, ws=ws)
        for k in range(10):
            flush()
            uzip.reduce_add(out[:total], outb[:tb], cb, n, C, out=outr, ws=ws, events=rev[k])
        torch.cuda.synchronize()
        t_red = float(np.mean([rev[k][0].elapsed_time(rev[k][3]) for k in range(10)]))
        t_red_k = float(np.mean([rev[k][0].elapsed_time(rev[k][1]) for k in range(10)]))
        trr, mr = uzip.stream_bytes(outr)
        _, mb = uzip.stream_bytes(outb)
        rb = stream_bytes_alg(n, C, m) + stream_bytes_alg(n, C, mb) + stream_bytes_alg(n, C, mr)
        reduce_hi = {"ms": round(t_red, 4), "k_reduce_tile_ms": round(t_red_k, 4),
                     "GBps_uncompressed_in": round(2 * 2 * n / (t_red * 1e-3) / 1e9, 1),
                     "algorithmic_bytes": rb, "op_frac": round(rb / (t_red * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "escape_rate_inputs": round(m / n, 6), "escape_rate_out": round(mr / n, 6),
                     "inputs": "the headline tensor and the same tensor with its K and V halves swapped "
                               "(a permutation: each input keeps its escape rate)"}
        del b, outb, outr
        reduce = reduce_config5(uzip, torch, dev, flush, C)

    # --- online calibration: codebook built on the device from the input
    # itself (whole input, or 256 KiB of every 2 MiB), then the encode ---
    online = None
    if not args.no_online:
        online = {}
        for label, blk, smp in (("whole_input", 0, 0), ("sample_256KiB_per_2MiB", 1 << 20, 1 << 17)):
            for _ in range(2):
                uzip.encode_online(x, C, blk, smp, out=out, ws=ws)
            oev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(10)]
            for row in oev:
                for e in row:
                    e.record()
            for k in range(10):
                flush()
                uzip.encode_online(x, C, blk, smp, out=out, ws=ws, events=oev[k])
            torch.cuda.synchronize()
            t_on = float(np.mean([oev[k][0].elapsed_time(oev[k][4]) for k in range(10)]))
            t_oncal = float(np.mean([oev[k][0].elapsed_time(oev[k][1]) for k in range(10)]))
            tot_on, m_on = uzip.stream_bytes(out)
            online[label] = {"ms": round(t_on, 4), "calibration_ms": round(t_oncal, 4),
                             "GBps": round(2 * n / (t_on * 1e-3) / 1e9, 1),
                             "slowdown_vs_offline_encode": round(t_on / t_enc, 3),
                             "escape_rate": round(m_on / n, 6), "ratio_total": round(2 * n / tot_on, 4)}
        uzip.encode(x, cb, C, out=out, ws=ws)      # leave the offline stream in place

    # --- ablation: Top-16 with positions against Top-15 + sentinel, Top-7
    # 3-bit + zero-point and Top-8 3-bit with positions, on the headline
    # tensor, under the offline codebook and one calibrated on the tensor
    # itself ---
    ablation = None
    if not args.no_ablation:
        ablation = {}
        cb_self = uzip.codebook_from_hist(uzip.histogram(x).cpu().numpy().astype(np.uint64))
        outs = torch.empty(uzip.s15_max_bytes(n, C), dtype=torch.uint8, device=dev)
        outz = torch.empty(uzip.z7_max_bytes(n, C), dtype=torch.uint8, device=dev)
        outt = torch.empty(uzip.t8_max_bytes(n, C), dtype=torch.uint8, device=dev)
        for label, cbx in (("offline_codebook", cb), ("self_calibrated_codebook", cb_self)):
            row = {}
            for fmt, enc_f, dec_f, buf in (("top16_positions", uzip.encode, uzip.decode, out),
                                           ("top15_sentinel", uzip.s15_encode, uzip.s15_decode, outs),
                                           ("top7_zero_point", uzip.z7_encode, uzip.z7_decode, outz),
                                           ("top8_3bit_positions", uzip.t8_encode, uzip.t8_decode, outt)):
                enc_f(x, cbx, C, out=buf, ws=ws)
                tt, mm = uzip.stream_bytes(buf)
                dec_f(buf, cbx, n, C, out=y, in_bytes=tt)
                torch.cuda.synchronize()
                if not torch.equal(y, x):
                    log(f"CORRECTNESS FAILURE ablation {label} {fmt}")
                    sys.exit(1)
                aev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(10)]
                for rr in aev:
                    for e in rr:
                        e.record()
                for k in range(10):
                    flush()
                    aev[k][0].record()
                    dec_f(buf, cbx, n, C, out=y, in_bytes=tt)
                    aev[k][1].record()
                    flush()
                    aev[k][2].record()
                    enc_f(x, cbx, C, out=buf, ws=ws)
                    aev[k][3].record()
                torch.cuda.synchronize()
                tdd = float(np.mean([aev[k][0].elapsed_time(aev[k][1]) for k in range(10)]))
                tee = float(np.mean([aev[k][2].elapsed_time(aev[k][3]) for k in range(10)]))
                row[fmt] = {"escape_rate": round(mm / n, 6), "ratio_total": round(2 * n / tt, 4),
                            "encode_ms": round(tee, 4), "decode_ms": round(tdd, 4),
                            "decode_GBps": round(2 * n / (tdd * 1e-3) / 1e9, 1)}
            for fmt in ("top15_sentinel", "top7_zero_point", "top8_3bit_positions"):
                row[fmt]["decode_slowdown"] = round(row[fmt]["decode_ms"] / row["top16_positions"]["decode_ms"], 3)
                row[fmt]["encode_slowdown"] = round(row[fmt]["encode_ms"] / row["top16_positions"]["encode_ms"], 3)
            ablation[label] = row
        del outs, outz, outt
        uzip.encode(x, cb, C, out=out, ws=ws)      # leave the headline stream in place

    # --- FP8 E5M2 variant on the same KV-cache recipe cast to E5M2 (2^28 bytes) ---
    fp8 = None
    if not args.no_fp8:
        log("fp8: generating the E5M2 KV cache")
        w8 = workloads.kv_cache_e5m2()
        x8 = torch.from_numpy(w8.x).to(dev)
        cb8 = uzip.fp8_calibrate(torch.from_numpy(w8.calib).to(dev))
        out8 = torch.empty(uzip.fp8_max_bytes(n, C), dtype=torch.uint8, device=dev)
        y8 = torch.empty_like(x8)
        uzip.fp8_encode(x8, cb8, C, out=out8, ws=ws)
        tot8, m8 = uzip.stream_bytes(out8)
        uzip.fp8_decode(out8, cb8, n, C, out=y8, in_bytes=tot8)
        torch.cuda.synchronize()
        if not torch.equal(y8, x8):
            log("CORRECTNESS FAILURE fp8 round trip")
            sys.exit(1)
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(10)]
        for row in fev:
            for e in row:
                e.record()
        for k in range(10):
            flush()
            uzip.fp8_encode(x8, cb8, C, out=out8, ws=ws, events=fev[k][:4])
            flush()
            uzip.fp8_decode(out8, cb8, n, C, out=y8, in_bytes=tot8, events=fev[k][4:])
        torch.cuda.synchronize()
        # whole-op durations from events around each call only
        oev8 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(10)]
        for row in oev8:
            for e in row:
                e.record()
        torch.cuda.synchronize()
        for k in range(10):
            flush()
            oev8[k][0].record()
            uzip.fp8_encode(x8, cb8, C, out=out8, ws=ws)
            oev8[k][1].record()
        torch.cuda.synchronize()
        te8 = float(np.mean([oev8[k][0].elapsed_time(oev8[k][1]) for k in range(10)]))
        td8 = float(np.mean([fev[k][4].elapsed_time(fev[k][5]) for k in range(10)]))
        nch = (n + C - 1) // C
        alg8 = n + (3 * n + 7) // 8 + (n + 1) // 2 + 3 * m8 + 4 * (nch + 1) + 256
        fp8 = {"workload": w8.name, "n": n, "escape_rate": round(m8 / n, 6),
               "ratio_payload": round(n / ((3 * n + 7) // 8 + (n + 1) // 2 + 3 * m8), 4),
               "ratio_total": round(n / tot8, 4),
               "encode_ms": round(te8, 4), "decode_ms": round(td8, 4),
               "encode_GBps": round(n / (te8 * 1e-3) / 1e9, 1), "decode_GBps": round(n / (td8 * 1e-3) / 1e9, 1),
               "op_roofline_frac": {"encode": round(alg8 / (te8 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                    "decode": round(alg8 / (td8 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
               "k8_encode_tile_ms": round(float(np.mean([fev[k][0].elapsed_time(fev[k][1]) for k in range(10)])), 4)}
        del x8, y8, out8

    # --- k-input fused reduce: one GPU's share of a two-shot all-reduce over
    # 8 GPUs (8 shards of 2^26 values, gradient recipe) ---
    reduce_k = None
    if not args.no_reduce_k:
        log("reduce_k: generating 8 shards of 2^26")
        ws_k = workloads.reduce_shards(8)
        nk = ws_k.x[0].size
        hist_k = None
        shards = []
        for r in ws_k.x:
            t = torch.from_numpy(r.view(np.int16)).to(dev)
            hist_k = uzip.histogram(t, hist_k)
            shards.append(t)
        cbk = uzip.codebook_from_hist(hist_k.cpu().numpy().astype(np.uint64))
        streams = []
        in_bytes = 0
        for t in shards:
            o = uzip.encode(t, cbk, C)
            tt, _ = uzip.stream_bytes(o)
            streams.append(o[:tt])
            in_bytes += tt
        del shards
        outk = torch.empty(uzip.max_bytes(nk, C), dtype=torch.uint8, device=dev)
        wsk = torch.empty(uzip.workspace_bytes(nk, C), dtype=torch.uint8, device=dev)
        for _ in range(3):
            uzip.reduce_k(streams, cbk, nk, C, out=outk, ws=wsk)
        kev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(10)]
        for row in kev:
            for e in row:
                e.record()
        for k in range(10):
            flush()
            uzip.reduce_k(streams, cbk, nk, C, out=outk, ws=wsk, events=kev[k])
        torch.cuda.synchronize()
        t_k = float(np.mean([kev[k][0].elapsed_time(kev[k][3]) for k in range(10)]))
        t_kt = float(np.mean([kev[k][0].elapsed_time(kev[k][1]) for k in range(10)]))
        out_bytes, mk = uzip.stream_bytes(outk)
        reduce_k = {"k": len(streams), "n_per_input": nk, "ms": round(t_k, 4), "k_reduce_k_tile_ms": round(t_kt, 4),
                    "GBps_uncompressed_in": round(len(streams) * 2 * nk / (t_k * 1e-3) / 1e9, 1),
                    "stream_roofline_frac": round((in_bytes + out_bytes) / (t_k * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                    "escape_rate_out": round(mk / nk, 6),
                    "inputs": f"{ws_k.name}: one GPU's share of a two-shot all-reduce over 8 GPUs"}
        del streams, outk, wsk

    res = {
        "metric": "encode/decode GB/s (uncompressed BF16) + ratio, 2^28-elt KV, 1 MI355X",
        "value": round(value, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u16", "data": "synthetic",
        "config": {"workload": f"{w.name}: BF16 KV cache {list(w.shape)} = {n} values, "
                               f"chunk {C}, codebook from layer 0 of another seed",
                   "n": n, "chunk": C},
        "encode_GBps": round(enc_gbps, 1), "decode_GBps": round(dec_gbps, 1),
        "encode_ms": round(t_enc, 4), "decode_ms": round(t_dec, 4),
        "ratio_payload": round(rho_payload, 4), "ratio_total": round(rho_total, 4),
        "escape_rate": round(m / n, 6), "coverage": round(1 - m / n, 6), "M": m,
        "stream_bytes": total, "calib_entropy_bits": round(entropy_bits(hist), 3),
        "calibrate_ms": round(t_cal * 1e3, 3),
        "B_hide_GBps": round(min(enc_gbps, dec_gbps) / rho_total, 1),
        "kernels_ms": {k: round(v, 4) for k, v in kern.items()},
        "encode_ms_stats": stats_ms(enc_list), "decode_ms_stats": stats_ms(dec_list),
        "op_roofline_frac": {k: round(v, 4) for k, v in op_frac.items()},
        "left_behind_ms": {**{k: round(v, 4) for k, v in behind.items()},
                           "what": "extra time of the next cache-evicting read after one call: the lines the call "
                                   "left dirty in the memory-side cache, written back then (median of 10)"},
        "op_roofline_frac_incl_left_behind": {k: round(v, 4) for k, v in op_frac_full.items()},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dom), "algorithmic_bytes": ab[dom],
                     "op": slow_op, "op_frac": round(op_frac[slow_op], 4),
                     "op_frac_incl_left_behind": round(op_frac_full[slow_op], 4)},
        "roofline_ops": roofline_ops,
        "copy_kernel_GBps": {"value": round(copy_gbps, 1), "frac_of_peak": round(copy_gbps / HBM_PEAK_GBPS, 4),
                             "what": "torch copy_ of 1 GiB to 1 GiB (2 GiB moved), median of 5 after a cache-evicting read"},
        "cache_flush_mib_before_each_call": args.flush_mib,
        "round_trip_bit_exact": round_trip, "oracle_stream_equal": parity,
        "reduce": reduce,
        "reduce_high_escape": reduce_hi,
        "reduce_k": reduce_k,
        "online_calibration": online,
        "fp8_e5m2": fp8,
        "ablation_formats": ablation,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(x_np, w.calib, C)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
