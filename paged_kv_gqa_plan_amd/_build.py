"""Build the gfx950 shared library ``libfl_paged_attn.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

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
OPT = "-O3"
# Per-source flags. The attention kernels never compute on a NaN: scores of keys past a
# request's end (whose pool rows may hold anything, NaN included) are replaced by -inf
# through index comparisons before any arithmetic reads them, and their V rows are zeroed
# with bit masks; so the compiler may treat every float there as a number, and max() then
# needs no quieting of signalling NaNs first (one VALU instruction less per operand). Host
# code elsewhere (the planner's and the RoPE call's argument checks) does test for NaN and
# keeps the default.
FILE_FLAGS = {"attn_kernels.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# Host-side sanitizers for a checking build of the host code (planner, allocator, entry
# points): every flag applies to the host compilation only, never to GPU code. Such a
# library is loaded with the sanitizer runtime preloaded (LD_PRELOAD) for the host tests.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_library(verbose: bool = False, out: str = LIB, defines=(), sources=None,
                  host_sanitize: bool = False) -> str:
    """Compile each source to an object (in parallel, with its own flags from FILE_FLAGS)
    and link them into the shared library `out`; host_sanitize: the checking build."""
    srcs = list(sources or SOURCES)
    san = HOST_SANITIZE if host_sanitize else []
    common = [hipcc(), f"--offload-arch={ARCH}", "-O1" if host_sanitize else OPT, "-std=c++17", "-fPIC",
              "-Wall", "-Wno-unused-function", *DEVICE_FLAGS, *san, *[f"-D{d}" for d in defines],
              "-I", INCLUDE, "-I", CSRC]
    noise = "is not a recognized feature for this target"

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
        if verbose and msgs.strip():
            print(msgs)

    with tempfile.TemporaryDirectory(prefix="fl_build_") as tmpdir:
        objs = [os.path.join(tmpdir, s + ".o") for s in srcs]
        cmds = [common + FILE_FLAGS.get(s, []) + ["-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(srcs, objs)]
        with ThreadPoolExecutor(max_workers=max(1, min(len(cmds), os.cpu_count() or 1, 16))) as ex:
            list(ex.map(run, cmds))
        tmp = out + ".tmp"
        run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *san, "-o", tmp])
        os.replace(tmp, out)
    return out


def build_probe(verbose: bool = False) -> str:
    return build_library(verbose, out=PROBE_LIB, sources=PROBE_SOURCES)


if __name__ == "__main__":
    import sys
    if len(sys.argv) == 3 and sys.argv[1] == "--host-sanitize":
        # the checking build, written to the path given (the in-tree library is left alone)
        print(build_library(verbose=True, out=os.path.abspath(sys.argv[2]), host_sanitize=True))
    else:
        print(build_library(verbose=True))
        print(build_probe(verbose=True))
