"""Build step of the C oracle: compiles oracle/c/rnl_oracle.c into
oracle/librnl_oracle.so with gcc (plain C, IEEE float, no contraction, no
fast-math, no vector intrinsics, no BLAS).  Run ``python -m
oracle.build_oracle`` or call :func:`build`."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c", "rnl_oracle.c")
LIB = os.path.join(HERE, "librnl_oracle.so")
FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread", "-Wall"]


def build(verbose: bool = False) -> str:
    cc = os.environ.get("CC") or shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler (gcc) found for the oracle")
    tmp = LIB + ".tmp"
    cmd = [cc, *FLAGS, SRC, "-o", tmp, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(" ".join(cmd))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
