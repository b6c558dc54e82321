"""Build the gfx950 shared library ``libpaged_attn.so`` in-tree with hipcc.

Usage: ``python -m paged_attention_decode_attn_amd.build`` (or
``__graft_entry__.build()``).  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpaged_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["pa_host.cpp", "pa_prefill_host.cpp", "pa_device.hip", "pa_cache.hip", "pa_prefill.hip", "pa_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    env = os.environ.get("HIPCC")
    if env:
        return env
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def build(verbose: bool = False) -> str:
    """Compile the library for gfx950 and return its path."""
    fd, tmp = tempfile.mkstemp(suffix=".so.tmp", dir=PKG)
    os.close(fd)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-I", INCLUDE,
           # no packed-FP32 VALU instructions in device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
        os.replace(tmp, LIB_PATH)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    build_cli(verbose)
    return LIB_PATH


CLI_SOURCE = os.path.join(PKG, "c_example", "pa_decode_cli.c")
CLI_PATH = os.path.join(PKG, "pa_decode_cli")


def build_cli(verbose: bool = False) -> str:
    """Compile the C caller of the library (plain C: the HIP runtime API for
    device memory, the library through paged_attn.h)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
           "-I", os.path.join(rocm, "include"), CLI_SOURCE, "-o", CLI_PATH,
           "-L", PKG, "-lpaged_attn", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stderr}")
    return CLI_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
