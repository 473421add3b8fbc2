"""Build libgdnbeam.so (HIP for gfx950) in-tree with hipcc.

    python linear_attention_beam_amd/build.py      # or __graft_entry__.build()

Packed fp32 VALU forms are switched off for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdnbeam.so")
SOURCES = ["gdn_beam_api.cpp", "gdn_step.hip", "gdn_select.hip", "gdn_fullstate.hip", "gdn_prefill.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", f"-I{os.path.join(ROOT, 'include')}", "-Wall",
              "-Wno-unused-variable", "-Wno-unused-function"]
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [cc, *common, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if verbose and err.strip():
            print(err, file=sys.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
