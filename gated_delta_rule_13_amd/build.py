"""Build the gfx950 HIP library ``libgdn.so`` in-tree with hipcc.

    python -m gated_delta_rule_13_amd.build [-v]

All device code is compiled for gfx950 only, with packed-fp32 instruction
selection disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
Each kernel family is its own translation unit (the fp16-operand kernel once
per (chunk, d_k) pair), compiled in parallel into objects under
``_build/`` and linked into one shared library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgdn.so")
ARCH = "gfx950"

# (chunk, d_k) pairs of the fp16-operand kernel; d_k 256 only up to 32-token
# chunks (the double-buffered key and query tiles of 64 would not fit in LDS);
# d_k 16 runs on the d_k 32 kernel, zero-padded
FAST_PAIRS = ([(c, d) for c in (16, 32, 64) for d in (16, 32, 64, 96, 128)] +
              [(16, 256), (32, 256)])


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def units() -> list[tuple[str, str, list[str]]]:
    """(object name, source, extra flags) of every translation unit."""
    out = [("gdn_api.o", "gdn_api.hip", []),
           ("gdn_inst_pipe.o", "gdn_inst_pipe.hip", []),
           ("gdn_inst_generic_bf16.o", "gdn_inst_generic.hip", ["-DGDN_GEN_BF16=1"]),
           ("gdn_inst_generic_f32.o", "gdn_inst_generic.hip", ["-DGDN_GEN_BF16=0"]),
           ("gdn_inst_rec.o", "gdn_inst_rec.hip", []),
           ("gdn_inst_seq.o", "gdn_inst_seq.hip", [])]
    for c, d in FAST_PAIRS:
        out.append((f"gdn_inst_fast_c{c}_d{d}.o", "gdn_inst_fast.hip", [f"-DGDN_C={c}", f"-DGDN_DK={d}"]))
    return out


NOISE = "is not a recognized feature for this target"


def _run(cmd: list[str]) -> tuple[int, str]:
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    return res.returncode, err


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(16, os.cpu_count() or 4)
    cmds = []
    objs = []
    for obj, src, extra in units():
        o = os.path.join(BUILD, obj)
        objs.append(o)
        cmds.append([hipcc(), *common_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", o])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, err) in zip(cmds, results):
        if rc != 0:
            raise RuntimeError("HIP build failed:\n" + " ".join(cmd) + "\n" + err)
        if verbose:
            print(" ".join(cmd), flush=True)
            if err.strip():
                print(err)
    tmp = LIB + f".tmp{os.getpid()}"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    rc, err = _run(link)
    if rc != 0:
        raise RuntimeError("HIP link failed:\n" + " ".join(link) + "\n" + err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
