"""Build liboracle.so (the plain CPU reference) with g++.

Test infrastructure: the flags keep every floating-point operation exactly
as written in oracle.cpp (no FMA contraction, no fast-math, no vector ISA
beyond the x86-64 baseline)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "oracle.cpp")

FLAGS = ["-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
         "-fno-tree-vectorize", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread"]


def build(verbose=False):
    cmd = ["g++", *FLAGS, SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_sanitized(verbose=False):
    """The same library built with AddressSanitizer and
    UndefinedBehaviorSanitizer (gcc runtimes) for the CPU test tier; returns
    its path.  Load it with gcc's libasan preloaded."""
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "liboracle_san.so")
    cmd = ["g++", *FLAGS, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", SRC, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
