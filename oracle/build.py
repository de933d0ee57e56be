"""Build the CPU oracle (plain C, gcc) into ``oracle/liboracle.so``.

Test infrastructure: only tests, the smoke check and the benchmark's
CPU-baseline leg load the result.  Compiled without fast-math and without
floating-point contraction so every operation rounds as written.
"""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = f"{LIB}.tmp{os.getpid()}"  # per process: concurrent test workers may build at once
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
