"""Build libgdnbeam.so (HIP for gfx950) in-tree with hipcc.

    python linear_attention_beam_amd/build.py      # or __graft_entry__.build()

Packed fp32 VALU forms are switched off for all device code.
"""
from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdnbeam.so")
SOURCES = ["gdn_beam_api.cpp", "gdn_step.hip", "gdn_select.hip", "gdn_fullstate.hip", "gdn_prefill.hip",
           "gdn_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


STEP_HASH = os.path.join(PKG, "step_kernel_code.sha")


def _elf_symbols(data: bytes):
    """(name, section index, value, size) of every symbol of a 64-bit little-endian ELF,
    and its section headers (addr, offset)."""
    import struct
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    secs = [struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize) for i in range(shnum)]
    out = []
    for sh in secs:
        if sh[1] != 2:                                   # SHT_SYMTAB
            continue
        strtab = secs[sh[6]]
        for k in range(sh[5] // 24):
            st_name, st_info, st_other, st_shndx, st_value, st_size = struct.unpack_from(
                "<IBBHQQ", data, sh[4] + 24 * k)
            end = data.index(b"\0", strtab[4] + st_name)
            out.append((data[strtab[4] + st_name:end].decode(), st_shndx, st_value, st_size))
    return out, secs


def step_kernel_code_hash(device_obj: str, d_k=None, d_v=None) -> str:
    """sha256[:16] of the step kernel's machine code: the instructions and kernel
    descriptor of every step_kernel instantiation (of head dims d_k x d_v when given), by
    name, from the gfx950 device object of gdn_step.hip.  The descriptor's bytes 16..23
    (the offset from the descriptor to the code, which moves when other kernels of the
    file change size) are left out; the rest of it holds the LDS, scratch and register
    counts.  It changes only when the compiled kernel does."""
    import hashlib
    data = open(device_obj, "rb").read()
    syms, secs = _elf_symbols(data)
    h = hashlib.sha256()
    tag = None if d_k is None else f"ILi{d_k}ELi{d_v}E"
    chosen = sorted(x for x in syms if "step_kernel" in x[0] and x[3] > 0 and (tag is None or tag in x[0]))
    for name, shndx, value, size in chosen:
        sec = secs[shndx]
        off = sec[4] + (value - sec[3])
        blob = data[off:off + size]
        if name.endswith(".kd"):
            blob = blob[:16] + blob[24:]
        h.update(name.encode())
        h.update(blob)
    return h.hexdigest()[:16]


def step_kernel_hashes(device_obj: str) -> dict:
    """{"all": hash of every instantiation, "<d_k>x<d_v>": hash of that head geometry's}"""
    syms, _ = _elf_symbols(open(device_obj, "rb").read())
    dims = sorted({(int(m.group(1)), int(m.group(2))) for x in syms if "step_kernel" in x[0]
                   for m in [re.search(r"step_kernelILi(\d+)ELi(\d+)E", x[0])] if m})
    out = {"all": step_kernel_code_hash(device_obj)}
    for dk, dv in dims:
        out[f"{dk}x{dv}"] = step_kernel_code_hash(device_obj, dk, dv)
    return out


def kernel_resources(device_obj: str) -> dict:
    """{kernel symbol: (LDS bytes, scratch bytes per lane)} from the kernel descriptors
    (the `.kd` symbols: group and private segment sizes, their first two words) of a
    gfx950 device object."""
    import struct
    data = open(device_obj, "rb").read()
    syms, secs = _elf_symbols(data)
    out = {}
    for name, shndx, value, size in syms:
        if name.endswith(".kd") and size >= 64:
            sec = secs[shndx]
            lds, scratch = struct.unpack_from("<II", data, sec[4] + (value - sec[3]))
            out[name[:-3]] = (lds, scratch)
    return out


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
    # the step kernel's device code on its own, for the hash that tells whether hardware
    # counters taken earlier still describe it
    dev = os.path.join(objdir, "gdn_step.gfx950.o")
    cmd = [cc, *common, f"--offload-arch={ARCH}", "--offload-device-only", "--no-gpu-bundle-output",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-c",
           os.path.join(CSRC, "gdn_step.hip"), "-o", dev]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"device compile failed: gdn_step.hip\n{r.stdout}\n{r.stderr}")
    with open(STEP_HASH, "w") as fh:
        json.dump(step_kernel_hashes(dev), fh, indent=1)
        fh.write("\n")
    # the prefill kernels' device code with the library's own flags, whose kernel
    # descriptors the host tests read (scratch memory of the chunk kernel)
    cmd = [cc, *common, f"--offload-arch={ARCH}", "--offload-device-only", "--no-gpu-bundle-output",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics", "-c",
           os.path.join(CSRC, "gdn_prefill.hip"), "-o", os.path.join(objdir, "gdn_prefill.gfx950.o")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"device compile failed: gdn_prefill.hip\n{r.stdout}\n{r.stderr}")
    # the selection kernels' device code, for the same checks (scratch memory)
    cmd = [cc, *common, f"--offload-arch={ARCH}", "--offload-device-only", "--no-gpu-bundle-output",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics", "-c",
           os.path.join(CSRC, "gdn_select.hip"), "-o", os.path.join(objdir, "gdn_select.gfx950.o")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"device compile failed: gdn_select.hip\n{r.stdout}\n{r.stderr}")
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
