"""Build libcoli.so (HIP kernels for gfx950 + host checks) in-tree with hipcc.

    python -m weight_streaming_gemv_qgemv_amd.build

Every translation unit compiles in parallel to an object under _build/, then
one hipcc link makes weight_streaming_gemv_qgemv_amd/libcoli.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INC = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libcoli.so")
BUILD = os.path.join(ROOT, "_build")

HIP_SOURCES = ["coli_gemv.hip", "coli_dec.hip", "coli_pre.hip", "coli_qmv.hip", "coli_idot.hip", "coli_router.hip", "coli_api.hip", "coli_stages.hip",
               "coli_tiled.hip"]
C_SOURCES = ["coli_validate.c"]

ARCH = os.environ.get("COLI_OFFLOAD_ARCH", "gfx950")

# Packed fp32 instructions stay off: the compiler emits plain fp32 FMAs.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffp-contract=fast", "-Wall", "-Wno-unused-result"]
C_FLAGS = ["-O2", "-std=c99", "-fPIC", "-Wall", "-Wextra"]


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libcoli")
    return p


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    procs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmd = [hipcc, *HIP_FLAGS, "-I", INC, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    for src in C_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmd = ["gcc", *C_FLAGS, "-I", INC, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append((cmd, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        msg = "\n\n".join(" ".join(c) + "\n" + t for c, t in failed)
        raise RuntimeError("libcoli build failed:\n" + msg)
    tmp = OUT + ".tmp"
    link = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("libcoli link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, OUT)
    return OUT


def build_validate_only(out_path: str) -> str:
    """The HIP-free host checks alone (for machines without ROCm devices)."""
    cmd = ["gcc", *C_FLAGS, "-shared", "-I", INC, "-I", CSRC,
           os.path.join(CSRC, "coli_validate.c"), "-o", out_path]
    subprocess.run(cmd, check=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
