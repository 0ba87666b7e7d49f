"""Build libtopo_attn.so in-tree with hipcc for gfx950 (no JIT, no torch extension machinery)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtopo_attn.so")
SOURCES = ["topo_api.hip", "topo_decode.hip", "topo_dense.hip", "topo_prefill.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions are not used (the host pass warns that it does not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I" + os.path.join(ROOT, "include"),
]


def build(verbose: bool = True, out: str = LIB) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed")
    if verbose:
        noise = "'-packed-fp32-ops' is not a recognized feature"
        for line in (res.stdout + res.stderr).splitlines():
            if line.strip() and noise not in line:
                print(line)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build()
