"""Build libpagedkv.so (HIP kernels + C ABI) for gfx950 with hipcc.

Each source compiles to an object in parallel; the objects link into
paged_kv_cache_193_amd/_lib/libpagedkv.so.  Always rebuilds.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libpagedkv.so")
OBJ_DIR = os.path.join(ROOT, "_build", "pagedkv")
SOURCES = ["api.cpp", "host_checks.cpp", "scheduler.cpp", "kv_append.hip", "decode.hip",
           "prefill.hip", "probe.hip"]
# host-only sources (no HIP): also built on their own with host sanitizers
HOST_SOURCES = ["host_checks.cpp", "scheduler.cpp"]
ARCH = "gfx950"

COMMON = [
    "-std=c++17", "-O3", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # packed fp32 (v_pk_*_f32) stays off in all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str, verbose: bool, defines=(), obj_dir=OBJ_DIR) -> str:
    obj = os.path.join(obj_dir, src + ".o")
    cmd = ["hipcc", *COMMON, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src),
           "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if verbose and errs.strip():
        print(errs, flush=True)
    return obj


def build(verbose: bool = False, defines=(), lib: str = LIB) -> str:
    """Compile every source and link `lib`.  `defines` (NAME=VALUE strings)
    override tuning constants; the default build uses none."""
    obj_dir = OBJ_DIR if not defines else os.path.join(
        OBJ_DIR, "_".join(d.replace("=", "") for d in defines))
    os.makedirs(obj_dir, exist_ok=True)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, defines, obj_dir), SOURCES))
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


def build_host_sanitized(lib: str, verbose: bool = False) -> str:
    """The host-only sources (scheduler, table checks, status text) as a
    shared library built by g++ with AddressSanitizer and
    UndefinedBehaviorSanitizer, for the CPU tests: no HIP, no device code."""
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-Wall", "-Wextra", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in HOST_SOURCES], "-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
