"""In-tree build of libkda.so for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_chunk.hip", "kda_chunk_bf16.hip",
           "kda_split_bf16.hip", "kda_segments.hip", "kda_layer.hip", "kda_bwd.hip",
           "kda_bwd_chunk.hip"]
HIPCC = "/opt/rocm/bin/hipcc"

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-fvisibility=hidden",
]


def build(verbose: bool = False, extra_flags=None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC] + FLAGS + (extra_flags or []) + ["-x", "hip"] + srcs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("libkda build failed:\n" + " ".join(cmd) + "\n" + r.stderr)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(" ".join(cmd))
        if r.stderr.strip():
            print("\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l))
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
