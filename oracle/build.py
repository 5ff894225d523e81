"""Build oracle/libssu_oracle.so with gcc (plain C, fp64, OpenMP, no FMA contraction).

TEST INFRASTRUCTURE ONLY.  Run as `python oracle/build.py`, or call build().
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "ssu_oracle.c"), os.path.join(HERE, "gdn_oracle.c")]
LIB = os.path.join(HERE, "libssu_oracle.so")


def build(verbose=False):
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-o", LIB + ".tmp"] + SRCS + ["-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
