"""Compile libfwd.so for gfx950 with hipcc (sources in csrc/, header in include/)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfwd.so")
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = ["gemm.hip", "attention.hip", "rows.hip", "decode.hip", "moe.hip", "fwd.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", INCLUDE, "-I", CSRC,
         # keep the compiler from emitting packed-fp32 VALU forms
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # fuse a*b+c into one fma only where it is written as one expression, so a
         # value's rounding does not depend on the code around it (e.g. on whether
         # its GEMM tile is cut by the last row)
         "-ffp-contract=on",
         "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops' is not a recognized feature" not in l)
        if verbose and text.strip():
            print(text, file=sys.stderr)
        if p.returncode != 0:
            failed.append((src, text))
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(f"--- {s}\n{t}" for s, t in failed))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB



def source_digest(files=("gemm.hip", "common.h", "kernels.h")) -> str:
    """sha256 over the GEMM kernel sources and the compile flags (ties stored counter
    data to the kernel it measured). Include paths enter relative to the repository
    root, so a copy of the tree elsewhere has the same digest."""
    import hashlib
    flags = [os.path.relpath(f, ROOT) if os.path.isabs(f) else f for f in FLAGS]
    h = hashlib.sha256(" ".join(flags).encode())
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    print(build(verbose=True))
