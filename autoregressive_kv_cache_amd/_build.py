"""Build the HIP library ``libkvc.so`` for gfx950 with hipcc (in-tree).

Run as ``python -m autoregressive_kv_cache_amd._build``.  The library is a
plain shared object with the C ABI of ``include/kvc.h``; it does not link
against PyTorch.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBRARY = os.path.join(PKG, "libkvc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no packed fp32 (v_pk_*_f32) instructions are generated.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]

SOURCES = [os.path.join(CSRC, "kvc_api.hip"), os.path.join(CSRC, "kvc_backward_api.hip"),
           os.path.join(CSRC, "kvc_measure.hip")]


def build(output: str = LIBRARY, extra: list[str] | None = None, verbose: bool = False) -> str:
    tmp = output + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to build libkvc.so")
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
