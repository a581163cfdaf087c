"""Builds the plain C++ oracle, oracle/liblcvq_oracle.so (test infrastructure only).

    python oracle/build_oracle.py

g++ -O2, C++17, OpenMP, no architecture-specific flags (the library is built here and
also loaded on other hosts). Building the checker is not using it: the GPU library never
loads this file's output.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lcvq_oracle.cpp")
LIB = os.path.join(HERE, "liblcvq_oracle.so")


def build():
    cxx = os.environ.get("CXX") or shutil.which("g++") or "g++"
    tmp = LIB + ".tmp"
    cmd = [cxx, "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", SRC, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + p.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
