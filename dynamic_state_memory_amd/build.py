"""Builds libdla.so (gfx950 HIP kernels + host C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = [os.path.join(PKG, "csrc", f) for f in ("dla_kernels.hip", "dla_prefill_rs.hip", "dla_abi.cpp")]
OUT = os.path.join(PKG, "_build", "libdla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("DLA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-x", "hip",
    # packed fp32 instructions stay off: plain fp32 arithmetic only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
    "-Wall", "-Wno-unused-result",
]


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, *FLAGS, *SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature; drop that note
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("hipcc failed building libdla.so")
    if out.strip() and verbose:
        print(out)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
