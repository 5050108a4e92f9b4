"""Compile libcq.so (HIP kernels + the C ABI of include/cq.h) for gfx950.

Every translation unit is compiled with hipcc for --offload-arch=gfx950 with
packed-FP32 instructions disabled and without fast-math (the Q8_0 quantizer
relies on correctly rounded fp32 division and round-to-nearest-even), then
linked into one shared library next to this file."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcq.so")
OBJ_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["cq_api.cpp", "quantize.hip", "gemv.hip", "gemv_mfma.hip", "gemm.hip", "moe.hip", "select.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src, verbose):
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


def build(verbose=False, jobs=8):
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_host_sanitized(verbose=False):
    """Debug build for the CPU test tier: cq_api.cpp (the argument validation
    of every entry point) compiled with AddressSanitizer and
    UndefinedBehaviorSanitizer on its host code, linked with the regular
    objects of the other translation units.  Needs build() first; returns
    the library path.  Load it with clang's ASan runtime preloaded."""
    objs = [os.path.join(OBJ_DIR, s + ".o") for s in SOURCES if s != "cq_api.cpp"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise FileNotFoundError(f"build() first: missing {missing}")
    san_obj = os.path.join(OBJ_DIR, "cq_api.cpp.san.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [HIPCC, *FLAGS, *san, "-x", "hip", "-c", os.path.join(CSRC, "cq_api.cpp"), "-o", san_obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the sanitized cq_api.cpp:\n" + r.stdout + r.stderr)
    out = os.path.join(OBJ_DIR, "libcq_hostsan.so")
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            san_obj, *objs, "-o", out]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True, capture_output=not verbose)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
