"""Host-side parts of bench.py, on the CPU: the one-GPU contract, the
algorithmic byte counts the roofline divides by, the HBM counter lookup that
turns itself off when the kernel source changes, and the CPU baseline leg."""
import importlib.util
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench(root=ROOT):
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(root, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                    # no JSON line for an unsupported N


@pytest.mark.parametrize("n,C", [(1, 64), (1001, 256), (65536, 1024), (100003, 4096)])
def test_algorithmic_bytes_bound_the_stream(n, C):
    # the compressed part of the byte count is the stream without its
    # 256-byte section padding: at most 5 gaps below the real stream size
    b = load_bench()
    x = workloads.random_words(n, 7)
    cb = oracle.calibrate(x[: max(1, n // 2)])
    s = oracle.encode(x, C, cb.dec)
    m = int(np.frombuffer(s[24:32].tobytes(), np.uint64)[0])
    ab = b.algorithmic_bytes(n, C, m)
    comp = ab["decode"] - 2 * n
    assert ab["encode"] == ab["decode"] == ab["k_decode_tile"]
    assert ab["k_encode_tile"] == 2 * n + n + (n + 1) // 2
    assert comp <= s.size < comp + 5 * 256
    assert comp - 4 * ((n + C - 1) // C + 1) - 256 == oracle.payload_bytes(n, m)


def test_traffic_lookup_follows_the_kernel_source(tmp_path):
    b = load_bench()
    got = b.measured_traffic("k_decode_tile")
    text = "".join(open(os.path.join(ROOT, "profiles", f)).read()
                   for f in os.listdir(os.path.join(ROOT, "profiles")) if f.endswith("_hbm_counters.md"))
    if got is not None:
        assert f"traffic_bytes k_decode_tile: {got}" in text
    # a copy of the tree whose kernel source differs reports no traffic
    for d in ("profiles", os.path.join("lossless_bf16_tensor_amd", "csrc")):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d)
    shutil.copy(os.path.join(ROOT, "bench.py"), tmp_path / "bench.py")
    with open(tmp_path / "lossless_bf16_tensor_amd" / "csrc" / "uzip.hip", "a") as f:
        f.write("\n// changed\n")
    assert load_bench(str(tmp_path)).measured_traffic("k_decode_tile") is None


def test_entropy_bits():
    b = load_bench()
    assert b.entropy_bits(np.ones(16, np.uint64)) == pytest.approx(4.0)
    h = np.zeros(256, np.uint64)
    h[7] = 10
    assert b.entropy_bits(h) == pytest.approx(0.0)


def test_cpu_baseline_leg():
    b = load_bench()
    w = workloads.config(1)
    r = b.cpu_baseline(w.x, w.calib, 1024, budget_s=1.0, sample=1 << 16)
    import os
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert r["cores"] == min(16, len(os.sched_getaffinity(0))) and r["one_thread"]["cores"] == 1
    assert r["streams_identical"] is True
    assert r["value"] > 0 and r["one_thread"]["value"] > 0 and "65536 values" in r["sample"]
    assert r["one_thread"]["histogram_GBps"] > 0
    # the round-trip rate is the harmonic combination of the two legs
    # (each figure is rounded to 4 decimals)
    assert r["value"] == pytest.approx(1 / (1 / r["encode_GBps"] + 1 / r["decode_GBps"]), abs=2e-4)
