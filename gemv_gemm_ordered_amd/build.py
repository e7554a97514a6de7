"""Build libggo.so: every HIP source compiled for gfx950 with hipcc.

Flags: -O3, contraction off (-ffp-contract=off plus a pragma in each ordered
source), no fast-math, binary32 denormals kept (the HIP default), packed
binary32 VALU ops disabled. The build info compiled into the library names
the target, the compiler, the flags and the SHA-256 of every source file.
"""
from __future__ import annotations

import hashlib
import json
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libggo.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["ordered_gemm.hip", "ordered_gemv.hip", "tree_gemv.hip", "mfma_invariant.hip", "mfma_gemv.hip", "capi.cpp", "freivalds.cpp", "cert_runtime.cpp"]
HEADERS = ["common.hpp", "kernels.hpp", "epilogue.hpp", os.path.join("..", "..", "include", "ggo.h")]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def build_info(csrc: str = CSRC) -> str:
    files = {os.path.normpath(s): _sha(os.path.join(csrc, s)) for s in SOURCES + HEADERS}
    try:
        ver = subprocess.run([HIPCC, "--version"], capture_output=True, text=True).stdout.splitlines()
        ver = [v for v in ver if "clang version" in v][:1]
    except OSError:
        ver = []
    return json.dumps({"arch": ARCH, "compiler": (ver or ["?"])[0], "flags": " ".join(FLAGS), "sources": files},
                      sort_keys=True)


def build(jobs: int = 8, csrc: str = CSRC, lib: str = LIB, build_dir: str = BUILD_DIR, only=None) -> str:
    """Compile every source of `csrc` (a copy of this package's csrc/ beside a copy of include/ serves
    too) into `build_dir` and link `lib`. With `only`, compile just those sources (capi.cpp, which
    carries the build info, always) and link the others' objects from this package's own build."""
    os.makedirs(build_dir, exist_ok=True)
    info = build_info(csrc)
    define = '-DGGO_BUILD_INFO="' + info.replace("\\", "\\\\").replace('"', '\\"') + '"'
    fresh = SOURCES if only is None else [s for s in SOURCES if s in set(only) | {"capi.cpp"}]

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, define, "-c", os.path.join(csrc, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(min(jobs, len(fresh))) as ex:
        built = dict(zip(fresh, ex.map(compile_one, fresh)))
    objs = [built[s] if s in built else os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in SOURCES]
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(*(int(a) for a in sys.argv[1:])))
