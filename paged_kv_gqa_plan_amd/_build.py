"""Build the gfx950 shared library ``libfl_paged_attn.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfl_paged_attn.so")
# benchmark-only measurement kernels (read floor, empty launch), a library of their own
PROBE_LIB = os.path.join(PKG, "libfl_read_probe.so")
PROBE_SOURCES = ["read_probe.hip"]
SOURCES = ["plan.cpp", "api.cpp", "page_pool.cpp", "attn_kernels.hip", "stage_copy.hip",
           "kv_append.hip", "kv_poison.hip", "kv_rope.hip", "noalloc.hip"]
ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of every kernel; MFMA accumulators live in ordinary
# VGPRs (the accumulator-register form costs a copy each time the VALU touches them); the
# attention kernel's first seven argument dwords (record, pools, kv heads) are preloaded
# into SGPRs at dispatch.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-mllvm", "-amdgpu-kernarg-preload-count=7"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build_library(verbose: bool = False, out: str = LIB, defines=(), sources=None) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function", *DEVICE_FLAGS, *[f"-D{d}" for d in defines],
           "-I", INCLUDE, "-I", CSRC, *[os.path.join(CSRC, s) for s in (sources or SOURCES)], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, out)
    return out


def build_probe(verbose: bool = False) -> str:
    return build_library(verbose, out=PROBE_LIB, sources=PROBE_SOURCES)


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_probe(verbose=True))
