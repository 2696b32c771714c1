"""Compile the C oracle into oracle/liboracle.so with gcc.

Test infrastructure: compiling the oracle does not put it on the product path.  Run directly
(``python oracle/build.py``) or through ``__graft_entry__.build()``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    # PA_ORACLE_LIB names an already-built variant of the oracle (used by the
    # test that plants mistakes in copies of the source to check the pins).
    override = os.environ.get("PA_ORACLE_LIB")
    if override:
        return override
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
