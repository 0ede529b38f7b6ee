"""Build the C oracle into oracle/liboracle.so with the host C compiler.

Test infrastructure only. The flags keep IEEE semantics exact: no contraction
of a*b+c into fused multiply-adds (the fp32 quantization steps must round
after every operation), no fast-math.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sage_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-frounding-math", "-Wall", "-Wextra"]


def build(verbose=False):
    cmd = [os.environ.get("CC", "gcc")] + CFLAGS + [SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
