"""Build libflce.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m linear_cross_entropy_fp32_amd.build [--verbose]

The library lands next to this file; the Python binding loads it from there.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libflce.so")
SOURCES = ["flce_kernels.hip", "ce_kernels.hip", "flce_api.cpp"]
ARCH = "gfx950"

# Packed fp32 VALU forms are kept off: hipcc would otherwise fuse pairs of
# fp32 ops into v_pk_* instructions.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libflce.so)")


def lds_dma_hazards(asm: str) -> list:
    """Inline-assembly LDS-DMA loads (buffer_load_* ... lds) that read an SGPR
    (the buffer descriptor, or M0) written by a VALU instruction (v_readlane,
    v_readfirstlane) fewer than five wait states earlier, or M0 written by a
    scalar instruction with no wait state in between: gfx950 needs those wait
    states and the compiler does not insert them in front of inline assembly.
    Returns one description per hazard found in the kernel assembly."""
    import re

    def sregs(tok):
        m = re.match(r"s\[(\d+):(\d+)\]$", tok)
        if m:
            return set(range(int(m.group(1)), int(m.group(2)) + 1))
        m = re.match(r"s(\d+)$", tok)
        return {int(m.group(1))} if m else set()

    out, func = [], "?"
    lines = asm.splitlines()
    for i, line in enumerate(lines):
        if re.match(r"^_Z\w+:", line):
            func = line.split(":")[0]
        s = line.strip()
        if not (s.startswith("buffer_load") and s.endswith(" lds")):
            continue
        used = sregs([o.strip() for o in s.split(None, 1)[1].split(",")][1]) | {"m0"}
        ws, j = 0, i - 1
        while j >= 0 and ws < 5:
            t = lines[j].strip()
            j -= 1
            if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
                continue
            if t.startswith("s_nop"):
                ws += int(t.split()[1], 0) + 1
                continue
            parts = t.split(None, 1)
            dst = parts[1].split(",")[0].strip() if len(parts) > 1 else ""
            written = {"m0"} if dst == "m0" else sregs(dst)
            if written & used and (parts[0].startswith("v_") or ("m0" in written and ws < 1)):
                out.append(f"{func}: '{s}' reads {dst} {ws} wait state(s) after '{t}'")
                break
            ws += 1
    return out


def build(verbose: bool = False, extra_flags=()) -> str:
    objs = []
    build_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [hipcc(), *HIP_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, *lang,
               "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    # the kernels' assembly, scanned for wait states that inline assembly needs
    asm_path = os.path.join(build_dir, "flce_kernels.s")
    cmd = [hipcc(), *HIP_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "--offload-device-only",
           "-S", os.path.join(CSRC, "flce_kernels.hip"), "-o", asm_path]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    with open(asm_path) as fh:
        hazards = lds_dma_hazards(fh.read())
    if hazards:
        raise RuntimeError("LDS-DMA wait-state hazards in the kernel assembly:\n  " +
                           "\n  ".join(hazards))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
