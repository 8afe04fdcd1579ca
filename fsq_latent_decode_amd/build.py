"""Build the HIP library in-tree: fsq_latent_decode_amd/lib/libfsq.so (gfx950).

    python -m fsq_latent_decode_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = ["csrc/api.hip", "csrc/append.hip", "csrc/decode.hip"]
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libfsq.so")
# a load-only kernel with the prefill append's traffic, for the benchmark's
# measurement of that kernel's load floor (not part of the FSQ library)
PROBE_SOURCES = ["csrc/probe_append_loads.hip"]
PROBE_LIB = os.path.join(LIB_DIR, "libfsq_probe.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile the library to `out` (the in-tree path by default); `defines`
    are extra -D macros of compile-time variants (A/B measurements). The
    in-tree build also compiles the benchmark's probe library."""
    if out == LIB:
        _compile(PROBE_SOURCES, PROBE_LIB, (), verbose)
    return _compile(SOURCES, out, defines, verbose)


def _compile(sources, out, defines, verbose) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Werror",
           # keep hipcc from emitting packed-fp32 VALU forms
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA accumulators in ordinary VGPRs: the decode kernels rescale
           # their accumulators with VALU ops, and with accumulation registers
           # the compiler copies every accumulator across each loop iteration
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-I", os.path.join(ROOT, "include"),
           "-o", tmp] + [f"-D{d}" for d in defines] + [os.path.join(PKG, s) for s in sources]
    res = subprocess.run(cmd, cwd=PKG, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
