"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer runs of the CPU
code: the fp64 oracle (plain C, gcc) and the argument validation of the C ABI
(the host part of ``gdn_api.hip``, clang; the device code is built as usual).
Each instrumented library is exercised in a child process that preloads the
matching sanitizer runtime, and any sanitizer report fails the test.  No GPU
is used: the oracle is CPU code, and every ABI call of ``tests/test_abi.py``
fails validation before a launch.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")

CHILD_ORACLE = r"""
import sys
sys.path.insert(0, {root!r})
import numpy as np
import oracle
from tests import oracle_pins
lib = oracle.load(path={path!r})
for pin in oracle_pins.ALL_PINS:
    pin(lambda *a, **kw: oracle.recurrent(*a, lib=lib, **kw))
# rejected arguments leave the outputs alone
null = oracle._ptr(None)
assert lib.gdn_oracle_recurrent_f64(0, 1, 1, 1, 1, null, null, null, null, null, null, null,
                                    null, null, 1) == -1
print("oracle ok")
"""


def run_child(code_or_args, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    args = [sys.executable] + (["-c", code_or_args] if isinstance(code_or_args, str) else code_or_args)
    res = subprocess.run(args, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    for r in REPORTS:
        assert r not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    from oracle.build import build_oracle
    path = build_oracle(out=str(tmp_path / "libgdn_oracle_san.so"), sanitize=True)
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                        text=True).stdout.strip()
    assert os.path.exists(rt), "gcc's libasan is missing"
    out = run_child(CHILD_ORACLE.format(root=ROOT, path=path), {"LD_PRELOAD": rt})
    assert "oracle ok" in out


def clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_validation_under_asan_ubsan(tmp_path):
    from gated_delta_rule_13_amd import build as gbuild
    rt = clang_asan_runtime()
    if rt is None or shutil.which(gbuild.hipcc()) is None:
        pytest.skip("no clang sanitizer runtime in this ROCm")
    objs = [o for o in (os.path.join(gbuild.BUILD, u[0]) for u in gbuild.units())
            if not o.endswith("gdn_api.o")]
    if not all(os.path.exists(o) for o in objs):
        gbuild.build()
    api = str(tmp_path / "gdn_api_san.o")
    cmd = [gbuild.hipcc(), f"--offload-arch={gbuild.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
           "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # instrument the host code only
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           f"-I{gbuild.INCLUDE}", f"-I{gbuild.CSRC}",
           "-c", os.path.join(gbuild.CSRC, "gdn_api.hip"), "-o", api]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    lib = str(tmp_path / "libgdn_san.so")
    res = subprocess.run([gbuild.hipcc(), f"--offload-arch={gbuild.ARCH}", "-shared", "-fPIC",
                          api, *objs, "-o", lib], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    out = run_child(["-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"],
                    {"LD_PRELOAD": rt, "GDN_TEST_LIB": lib, "HIP_VISIBLE_DEVICES": ""})
    assert " passed" in out and " failed" not in out, out[-3000:]
