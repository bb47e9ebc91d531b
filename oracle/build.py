"""Build the fp64 CPU oracle library (test infrastructure only).

``build_oracle()`` compiles ``gdn_oracle.c`` with gcc into
``oracle/libgdn_oracle.so``.  ``build_oracle(src=..., out=...)`` compiles
another source file (a copy with a planted mistake, written by the test that
checks that the oracle's pins catch such mistakes) to another path.
``sanitize=True`` adds AddressSanitizer and UndefinedBehaviorSanitizer (host
code only; used by the sanitizer test).
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")


def library_path() -> str:
    return os.path.join(HERE, "libgdn_oracle.so")


def build_oracle(src: str = SRC, out: str | None = None, quiet: bool = True,
                 sanitize: bool = False) -> str:
    """Compile the oracle; returns the path of the shared library."""
    out = out or library_path()
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        # keep IEEE fp64 semantics: no fast-math, no contraction into FMA
        "-ffp-contract=off",
        "-Wall", "-Wextra",
    ]
    if sanitize:
        cmd += ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                "-fno-sanitize-recover=undefined"]
    cmd += [src, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    if not quiet and res.stderr:
        print(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle(quiet=False))
