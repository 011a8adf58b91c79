"""Build the CPU oracle (plain C, gcc) into oracle/libkin_oracle.so.

Test infrastructure: the oracle is built so the tests, the smoke check and
the benchmark's CPU baseline can call it; nothing in the product path loads
it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kin_oracle.c")
LIB = os.path.join(HERE, "libkin_oracle.so")

# -ffp-contract=off: every product and sum is rounded on its own, exactly as
# the C source reads; no fused multiply-add is introduced behind its back.
CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
