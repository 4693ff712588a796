"""Build libdcasparse.so (gfx950) in-tree with hipcc.

Usage: python -m sparse_dual_chunk_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdcasparse.so")
SOURCES = ["api.hip", "rope.hip", "attn.hip", "decode.hip", "vs_score.hip", "select.hip", "sequence.hip", "moe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms stay off: the compiler would otherwise form them by itself
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wno-unused-result",
]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + [f"-D{d}" for d in defines] + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libdcasparse.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
