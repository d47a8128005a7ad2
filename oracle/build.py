"""Build the CPU oracle (test infrastructure) as oracle/liboracle.so with gcc.

Plain C11 with GCC's __int128; -O2 -ffp-contract=off and no fast-math, so every binary32
add is a single IEEE add with the default rounding and no flush-to-zero.  `mutant` builds a
variant with one deliberate mistake, used only by the oracle's own pin tests.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")


def lib_path(mutant: int = 0) -> str:
    if mutant:
        return os.path.join(HERE, "_build", f"liboracle_m{mutant}.so")
    # a separately built variant of the same source (the sanitized build below) when named
    return os.environ.get("QG_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")


def build(mutant: int = 0, quiet: bool = True) -> str:
    out = lib_path(mutant)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["gcc", "-std=gnu11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wno-unused-function", f"-DOR_MUTANT={mutant}",
           SRC, "-o", out + ".tmp", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("oracle build failed: " + " ".join(cmd))
    os.replace(out + ".tmp", out)
    if not quiet:
        print("built", out)
    return out


def build_sanitized(out: str) -> str:
    """The unchanged oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (every
    finding fatal), for a test that runs the pins against it; load it with libasan preloaded
    and QG_ORACLE_LIB naming it."""
    cmd = ["gcc", "-std=gnu11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-Werror", "-Wno-unused-function", "-DOR_MUTANT=0", SRC, "-o", out, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("sanitized oracle build failed: " + " ".join(cmd))
    return out


if __name__ == "__main__":
    build(quiet=False)
