"""Build the gfx950 shared library libvdn_hybrid_attn.so in-tree with hipcc.

Every source is compiled to an object of its own (in parallel, in a temporary
directory) with the flags below plus any per-file flags, then the objects are
linked into the library next to this file.

Usage: python -m hybrid_sparse_linear_chunked_amd.build   (or call build()).
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libvdn_hybrid_attn.so")
SOURCES = ["api.cpp", "attn.hip", "attn64.hip", "vda.hip", "proj.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # hipcc -O3 forms packed fp32 instructions on its own; keep them off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no NaNs flow through the kernels: lets max/min skip NaN-quieting copies
    "-fno-honor-nans", "-mno-amdgpu-ieee",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]
# attn64.hip: MFMA results in ordinary VGPRs (its scores feed the softmax on the
# VALU; its P.V accumulators are placed in the accumulation registers by hand)
PER_FILE = {"attn64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the library; returns its path."""
    with tempfile.TemporaryDirectory(prefix="vdn_build_") as tmpdir:
        procs, objs = [], []
        for s in SOURCES:
            src = os.path.join(CSRC, s)
            obj = os.path.join(tmpdir, s + ".o")
            cmd = [HIPCC] + FLAGS + PER_FILE.get(s, []) + ["-c"]
            cmd += (["-x", "hip", src] if s.endswith(".cpp") else [src]) + ["-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for s, p in procs:
            out, _ = p.communicate()
            if p.returncode != 0:
                sys.stderr.write(out)
                failed.append(s)
        if failed:
            raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed linking libvdn_hybrid_attn.so")
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
