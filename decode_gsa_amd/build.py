"""Build libgsa.so (HIP for gfx950) in-tree: ``python -m decode_gsa_amd.build``."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgsa.so")

ARCH = "gfx950"
# -packed-fp32-ops: keep hipcc from emitting packed fp32 VALU ops.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


STAMPS_LIB = os.path.join(PKG, "libgsa_stamps.so")


def build(verbose: bool = False, stamps: bool = False) -> str:
    """Compile every source under csrc/ into decode_gsa_amd/libgsa.so; returns
    its path. stamps=True builds the diagnostic libgsa_stamps.so instead (the
    decode kernel records its phase edges; bench.py --phase-stamps reads
    them)."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    out_dir = os.path.join(ROOT, "_build", "stamps" if stamps else "")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    procs = []
    extra = ["-DGSA_PHASE_STAMPS"] if stamps else []
    for s in srcs:
        o = os.path.join(out_dir, os.path.basename(s) + ".o")
        lang = ["-x", "hip"] if s.endswith(".hip") else []
        cmd = [hipcc()] + HIP_FLAGS + extra + ["-I", INCLUDE, "-I", CSRC] + lang + ["-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(o)
    failed = []
    for s, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        msgs = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((s, msgs))
        elif verbose and msgs.strip():
            print(msgs)
    if failed:
        for s, m in failed:
            sys.stderr.write(f"--- {s}\n{m}\n")
        raise RuntimeError("libgsa build failed: " + ", ".join(os.path.basename(s) for s, _ in failed))
    lib = STAMPS_LIB if stamps else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, stamps="--stamps" in sys.argv))
