"""Build the gfx950 HIP library (libkda.so) in-tree with hipcc.

    python -m linear_attention_kda_amd.build [--verbose]

Every build recompiles from source.  The library is written next to this file
and loaded by the Python binding from there.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = [os.path.join(CSRC, f) for f in
           ("kda_api.cpp", "kda_fwd_kernel.hip", "kda_gdn_kernel.hip", "kda_fwd_dim.hip",
            "kda_decode_kernel.hip", "kda_bwd.hip", "kda_noalloc.hip", "kda_fwd_hd64_kernel.hip")]
ARCH = "gfx950"

# Packed-fp32 VALU instructions are disabled for all device code; the host pass
# warns that it does not know the feature, which is harmless.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-I", os.path.join(ROOT, "include"),
           *SOURCES, "-o", tmp, *(extra or [])]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (proc.stdout + proc.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
