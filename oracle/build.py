"""Build the CPU oracle: plain gcc, contraction off, no fast-math.

TEST INFRASTRUCTURE ONLY (the oracle is used by the tests, the smoke check and
the benchmark's CPU-baseline leg, never by the library).

The SHA-256 of the source file is compiled into the library
(``oracle_source_sha256``), so a test can show which file a build read; the
mutant gates build a copied, modified source through this same function.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-unsafe-math-optimizations",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def sha256_file(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def build(src: str = SRC, out: str = LIB, extra: list[str] | None = None) -> str:
    digest = sha256_file(src)
    cmd = ["gcc", *CFLAGS, f'-DORACLE_SRC_SHA256="{digest}"', *(extra or []), src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:]))
