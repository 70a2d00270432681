"""Builds libfusednorm.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m residual_add_rmsnorm_amd._build

hipcc cross-compiles without a GPU. Packed fp32 instructions are disabled for
all device code (``-packed-fp32-ops``); the host pass warns that it does not
know that feature, which is harmless. Host code is built with hidden default
visibility, so the shared library exports exactly the functions that
include/fusednorm.h marks with FUSEDNORM_API.
"""
import os
import re
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfusednorm.so")
SOURCES = [os.path.join(CSRC, "fusednorm_kernels.hip"), os.path.join(CSRC, "fusednorm_api.cpp"),
           os.path.join(CSRC, "fusednorm_launch_policy.cpp"), os.path.join(CSRC, "fusednorm_stream.hip")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-fvisibility=hidden", "-Xarch_host", "-fvisibility-inlines-hidden",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def exported_functions(header: str = os.path.join(INCLUDE, "fusednorm.h")) -> list:
    """Names of the functions the public header marks with FUSEDNORM_API."""
    with open(header) as f:
        text = f.read()
    return re.findall(r"^FUSEDNORM_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M)


def version_script(path: str) -> str:
    """A linker version script that exports the header's functions and hides
    every other symbol (the compiler's own per-file data symbols included)."""
    names = exported_functions()
    with open(path, "w") as f:
        f.write("{\n  global:\n")
        for n in names:
            f.write(f"    {n};\n")
        f.write("  local:\n    *;\n};\n")
    return path


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    tmpdir = tempfile.mkdtemp(prefix="fusednorm_build_")
    vs = version_script(os.path.join(tmpdir, "exports.map"))
    cmd = [hipcc(), *HIPCC_FLAGS, f"-Wl,--version-script={vs}", *extra_flags, *SOURCES,
           "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        r = subprocess.run(cmd, capture_output=True, text=True)
    finally:
        os.remove(vs)
        os.rmdir(tmpdir)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
