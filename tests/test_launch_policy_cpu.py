"""The launch-shape pickers on the CPU: compiled as plain host C++ with their
own source file, called for every row width the library accepts, 1 to 16
partials and token counts on both sides of each rule boundary, on devices of
80, 256 and 304 CUs. Every shape must be one the kernels are compiled for
(vectors per lane, partials per load chunk, workgroup size within the
variant's bound, whole waves) and cover the row, and the persistent grid must
be chosen exactly where the rule says (rows of at least 896 vectors, more
tokens than CUs and at most 8 per CU). For rows of whole 1x128 groups there
must be a lane per group and the groups must fit the LDS row that the block
FP8 epilogue stores its scales from."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "residual_add_rmsnorm_amd", "csrc")


def _compiler():
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++"), shutil.which("g++")):
        if c and os.path.exists(c):
            return c
    pytest.skip("no host C++ compiler")


def test_every_launch_shape_is_valid_and_follows_the_rule(tmp_path):
    exe = tmp_path / "shape_rule_check"
    cmd = [_compiler(), "-std=c++17", "-O1", "-x", "c++", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(ROOT, "tests", "host", "shape_rule_check.cpp"),
           os.path.join(CSRC, "fusednorm_launch_policy.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-2000:] + r.stderr[-2000:]
