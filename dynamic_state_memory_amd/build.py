"""Builds libdla.so (gfx950 HIP kernels + host C ABI) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = [os.path.join(PKG, "csrc", f) for f in ("dla_kernels.hip", "dla_prefill_rs.hip", "dla_state_score.hip", "dla_abi.cpp")]
OUT = os.path.join(PKG, "_build", "libdla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("DLA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-x", "hip",
    # packed fp32 instructions stay off: plain fp32 arithmetic only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
    "-Wall", "-Wno-unused-result",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature; drop that note
    return r.returncode, "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel: each keeps its kernels
    and their launchers together, so no device code links across objects),
    then link libdla.so."""
    bdir = os.path.dirname(OUT)
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.splitext(os.path.basename(f))[0] + ".o") for f in SRC]
    cmds = [[HIPCC, *FLAGS, "-c", src, "-o", obj] for src, obj in zip(SRC, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with cf.ThreadPoolExecutor(len(cmds)) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, out), c in zip(results, cmds):
        if rc != 0:
            sys.stderr.write(out + "\n")
            raise RuntimeError(f"hipcc failed compiling {c[-3]}")
        if out.strip() and verbose:
            print(out)
    tmp = OUT + ".tmp"
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    rc, out = _run(link)
    if rc != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("hipcc failed linking libdla.so")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
