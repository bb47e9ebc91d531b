"""Build the fp64 CPU oracle library (test infrastructure only).

``build_oracle()`` compiles ``gdn_oracle.c`` with gcc into
``oracle/libgdn_oracle.so``.  ``build_oracle(mutant=n, out_dir=...)`` builds
a copy that carries planted mistake ``n``; only the test that checks that the
oracle's pins catch such mistakes asks for one.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")


def library_path(mutant: int = 0, out_dir: str | None = None) -> str:
    out_dir = out_dir or HERE
    name = "libgdn_oracle.so" if mutant == 0 else f"libgdn_oracle_mutant{mutant}.so"
    return os.path.join(out_dir, name)


def build_oracle(mutant: int = 0, out_dir: str | None = None, quiet: bool = True) -> str:
    """Compile the oracle; returns the path of the shared library."""
    out = library_path(mutant, out_dir)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        # keep IEEE fp64 semantics: no fast-math, no contraction into FMA
        "-ffp-contract=off",
        "-Wall", "-Wextra",
        f"-DGDN_ORACLE_MUTANT={int(mutant)}",
        SRC, "-o", tmp,
    ]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    if not quiet and res.stderr:
        print(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle(quiet=False))
