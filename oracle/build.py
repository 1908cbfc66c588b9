"""Compile the C oracle (test infrastructure: the forward recurrence and its gradients) with gcc
into oracle/libkda_oracle.so."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
# (source, optimisation level): the forward keeps the level its CPU-baseline figures were
# measured with; the backward, run only by the full-size GPU tests, is built for speed
SRCS = [(os.path.join(HERE, "kda_oracle.c"), "-O2"), (os.path.join(HERE, "kda_oracle_bwd.c"), "-O3")]
LIB = os.path.join(HERE, "libkda_oracle.so")


def build(verbose: bool = False) -> str:
    objs = []
    for src, opt in SRCS:
        obj = os.path.join(HERE, os.path.basename(src) + ".o")
        cmd = ["gcc", opt, "-std=c11", "-fPIC", "-pthread", "-Wall", "-Wextra", "-c", src,
               "-o", obj]
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
        objs.append(obj)
    cmd = ["gcc", "-shared", "-pthread", *objs, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    for obj in objs:
        os.remove(obj)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
