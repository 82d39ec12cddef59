"""Builds the CPU oracle (test infrastructure) with gcc: plain C, OpenMP over
independent rows/tokens, -O2 and no -ffast-math, so every sum keeps its written
order."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libmoe_oracle.so")


def build_oracle(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "moe_oracle.c")
    out = library_path()
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_variant(edits, out_dir: str) -> str:
    """Compile a copy of the oracle source with textual edits [(old, new), ...]
    applied, into out_dir. Used only by tests that plant a mistake in the oracle
    to show that its pins catch it; the default build is never modified."""
    with open(os.path.join(_HERE, "moe_oracle.c")) as f:
        text = f.read()
    for old, new in edits:
        if old not in text:
            raise ValueError(f"edit target not found in oracle source: {old!r}")
        text = text.replace(old, new, 1)
    src = os.path.join(out_dir, "moe_oracle_variant.c")
    with open(src, "w") as f:
        f.write(text)
    out = os.path.join(out_dir, "libmoe_oracle_variant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                    "-ffp-contract=off", "-w", "-o", out, src, "-lm"], check=True)
    return out


if __name__ == "__main__":
    print(build_oracle(verbose=True))
