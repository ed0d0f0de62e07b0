"""Builds the C++ oracle (oracle/nanospec_oracle.cpp) into
oracle/libnanospec_oracle.so with g++ and OpenMP.  Test infrastructure: the
library is loaded by tests/ and by bench.py's cpu_baseline leg only.

Products and sums are kept in plain float64 (-ffp-contract=off: no fused
multiply-add), so each logit is the sequential sum of its definition."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nanospec_oracle.cpp")
LIB = os.path.join(HERE, "libnanospec_oracle.so")
FLAGS = ["-O3", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]


def build() -> str:
    tmp = LIB + ".tmp"
    p = subprocess.run(["g++", *FLAGS, SRC, "-o", tmp], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"g++ failed:\n{p.stdout}")
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    """The library's path, building it only when it is missing."""
    return LIB if os.path.exists(LIB) else build()


if __name__ == "__main__":
    print(build())
