"""Build the gfx950 shared library libgptq_mi355x.so in-tree with hipcc.

    python -m post_weight_quantization_23_amd.build [--jobs N] [--verbose] [--incremental]

Every HIP source under csrc/ is compiled for gfx950 only, with packed fp32
instructions disabled, and linked into one shared library exposing the C ABI
declared in include/gptq.h.  The library carries the SHA-256 of the sources it
was built from (`gptq_build_id()`), which the loader compares with the sources
beside it.  --incremental recompiles only the objects whose source, headers or
flags changed (the default rebuilds everything).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libgptq_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

# slowest first: the pool starts them at once
SOURCES = ["quantize.hip", "linear.hip", "gemm_f32.hip", "syrk.hip", "gemv.hip", "prepare.hip",
           "hadamard.hip", "pack.hip", "gptq_api.hip", "workspace.hip"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


HEADERS = [os.path.join(CSRC, "common.hpp"), os.path.join(CSRC, "kernels.hpp")]
API_HEADER = os.path.join(ROOT, "include", "gptq.h")   # included by gptq_api.hip only


def source_id() -> str:
    """SHA-256 over every file the library is built from (names and contents)."""
    h = hashlib.sha256()
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp")))
    files.append(os.path.join(ROOT, "include", "gptq.h"))
    for path in files:
        h.update(os.path.relpath(path, ROOT).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _object_key(src: str) -> str:
    h = hashlib.sha256(" ".join(COMMON_FLAGS).encode())
    for path in [os.path.join(CSRC, src), *HEADERS, *([API_HEADER] if src == "gptq_api.hip" else [])]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the gfx950 library cannot be built")
    return path


def _compile(src: str, verbose: bool, incremental: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    stamp = obj + ".key"
    key = _object_key(src)
    if incremental and os.path.exists(obj) and os.path.exists(stamp):
        with open(stamp) as f:
            if f.read() == key:
                return obj
    cmd = [hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    warn = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if verbose and warn:
        print(warn, flush=True)
    with open(stamp, "w") as f:
        f.write(key)
    return obj


def _compile_build_id(sid: str, verbose: bool) -> str:
    """A host-only object whose gptq_build_id() returns the sources' SHA-256."""
    src = os.path.join(BUILD_DIR, "build_id.cpp")
    obj = os.path.join(BUILD_DIR, "build_id.o")
    with open(src, "w") as f:
        f.write('extern "C" const char* gptq_build_id(void) { return "%s"; }\n' % sid)
    cmd = ["g++", "-O2", "-fPIC", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"g++ failed on build_id.cpp:\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False, incremental: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    sid = source_id()   # taken before compiling: a source edited meanwhile makes the library stale, not mislabelled
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, incremental), SOURCES))
    objs.append(_compile_build_id(sid, verbose))
    tmp = LIB_PATH + ".tmp"
    # --no-undefined: a kernel the host pass failed to instantiate must fail the
    # build here, not the load of the library
    cmd = [hipcc(), "-shared", "--offload-arch=gfx950", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--incremental", action="store_true",
                    help="recompile only objects whose source, headers or flags changed")
    args = ap.parse_args(argv)
    path = build(args.jobs, args.verbose, args.incremental)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
