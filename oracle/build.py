"""Compile oracle.c into oracle/liboracle.so with the host C compiler.

The oracle is test infrastructure: a plain single-threaded C build, no
vectorisation flags, no OpenMP, nothing tuned.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def compile_source(src: str, out: str, verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    return compile_source(SRC, LIB, verbose)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
