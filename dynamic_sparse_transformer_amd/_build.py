"""Build libtopo_attn.so in-tree with hipcc for gfx950 (no JIT, no torch extension machinery).

Each source is compiled to an object file on its own (in parallel), then the objects are linked
into the shared library. Every kernel is defined and launched in the same source file, so no
relocatable device code is needed.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtopo_attn.so")
OBJDIR = os.path.join(ROOT, "_build")
SOURCES = ["topo_api.hip", "topo_decode.hip", "topo_dense.hip", "topo_prefill.hip", "topo_noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are not used (the host pass warns that it does not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I" + os.path.join(ROOT, "include"),
]
NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    return res.returncode, res.stdout + res.stderr


def build(verbose: bool = True, out: str = LIB) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = list(SOURCES)
    objs = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o") for s in srcs]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    failed = False
    for (rc, text), s in zip(results, srcs):
        lines = [ln for ln in text.splitlines() if ln.strip() and NOISE not in ln]
        if rc != 0:
            failed = True
            sys.stderr.write(f"--- {s}\n" + "\n".join(lines) + "\n")
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = out + ".tmp"
    rc, text = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    if rc != 0:
        sys.stderr.write(text)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build()
