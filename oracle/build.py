"""Build the CPU oracle (oracle/ne_oracle.c) into oracle/libne_oracle.so.

Test infrastructure only: the product library never links or loads it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ne_oracle.c")
LIB = os.path.join(HERE, "libne_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc -O2 -fopenmp; returns the library path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
