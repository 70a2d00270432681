"""Builds libfusednorm.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m residual_add_rmsnorm_amd._build

hipcc cross-compiles without a GPU. Packed fp32 instructions are disabled for
all device code (``-packed-fp32-ops``); the host pass warns that it does not
know that feature, which is harmless.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfusednorm.so")
SOURCES = [os.path.join(CSRC, "fusednorm_kernels.hip"), os.path.join(CSRC, "fusednorm_api.cpp"),
           os.path.join(CSRC, "fusednorm_stream.hip")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, *SOURCES, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
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
