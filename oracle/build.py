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


def build_sanitized(out: str, verbose: bool = False) -> str:
    """oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer (gcc),
    for the CPU tests of the sanitizer build; same source, same arithmetic."""
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-Wall",
           "-Wextra", SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
