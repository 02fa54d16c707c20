"""Build the CPU oracle (plain C, gcc) into oracle/libsp_oracle.so.

Test infrastructure only: the oracle is built so that the tests, the smoke
check and the bench's CPU-baseline leg can call it; the product path never
loads it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sp_oracle.c")
LIB = os.path.join(HERE, "libsp_oracle.so")

# -ffp-contract=off: no fused multiply-add, so every fp32 operation rounds once,
# in the order the source writes it.  No -ffast-math.
CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def build(verbose=False):
    """Compile the oracle; always recompiles.  Returns the library path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
