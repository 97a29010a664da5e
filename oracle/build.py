"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, no fast-math and no FMA contraction, so every fp32 operation in
mbt_oracle.c rounds exactly as written.  `mutation` builds a copy with one
planted mistake (used only by the tests that prove the pins can fail).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mbt_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-fno-builtin", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
          "-Wno-maybe-uninitialized"]


def build(out=LIB, mutation=0, extra=()):
    cmd = ["gcc", *CFLAGS, f"-DMBT_ORACLE_MUTATION={int(mutation)}", *extra,
           SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
