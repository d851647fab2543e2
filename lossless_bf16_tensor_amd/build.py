"""Build the HIP library libuzip.so in-tree for gfx950 with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "uzip.hip")
LIB = os.path.join(HERE, "libuzip.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


# Host code only under AddressSanitizer and UndefinedBehaviorSanitizer (the
# device code is built as usual): for CPU tests of the host-side stream
# parsing, validation and table building. The process that loads such a
# build must preload clang's ASan runtime.
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-g",
]


def build(verbose: bool = False, sanitize: bool = False, out: str | None = None) -> str:
    lib = out or LIB
    cmd = [HIPCC, *FLAGS, *(SANITIZE_FLAGS if sanitize else []), "-I", os.path.join(ROOT, "include"),
           "-o", lib + ".tmp", SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    if verbose:
        print(r.stderr)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
