"""Build libwise.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m block_sparse_paged_split_amd.build
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = ["wise_api.hip", "wise_split.hip", "wise_finish.hip", "wise_pages.hip", "wise_state.hip"]
LIB = os.path.join(PKG, "libwise.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: ROCm is required to build libwise")


def command(out: str = LIB, extra=(), sources=SOURCES):
    src = [os.path.join(PKG, "csrc", s) for s in sources]
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 instructions are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
            *extra, *src, "-o", out]


# The benchmark's read-ceiling probe (not part of libwise; only bench.py loads it).
PROBE_SOURCES = ["read_probe.hip"]
PROBE_LIB = os.path.join(PKG, "libwise_probe.so")


def _compile(cmd, out, verbose):
    tmp = out + ".tmp"
    cmd = [tmp if c == out else c for c in cmd]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build of {os.path.basename(out)} failed")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _compile(command(LIB), LIB, verbose)
    _compile(command(PROBE_LIB, sources=PROBE_SOURCES), PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
