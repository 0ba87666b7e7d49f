"""The C-ABI library without a GPU: it loads, exports every entry point that include/topo_attn.h
declares, agrees with the binding on the parameter struct layout, and rejects bad arguments on the
host before anything is launched (no compute calls here)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import dynamic_sparse_transformer_amd as topo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "topo_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(topo_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = topo.load_library()
    names = declared_functions()
    assert set(names) == set(topo.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_params_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "topo_attn.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(topo_params_t), offsetof(topo_params_t, n_ctx),
         offsetof(topo_params_t, q_pos0), offsetof(topo_params_t, W), offsetof(topo_params_t, softmax_scale),
         offsetof(topo_params_t, dtype), offsetof(topo_params_t, flags), offsetof(topo_params_t, causal));
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    P = topo.TopoParams
    want = [ctypes.sizeof(P), P.n_ctx.offset, P.q_pos0.offset, P.W.offset, P.softmax_scale.offset, P.dtype.offset,
            P.flags.offset, P.causal.offset]
    assert got == want


def _p(**kw):
    base = dict(B=1, Hq=32, Hkv=8, d=128, n_ctx=1 << 20, n_q=1, q_pos0=(1 << 20) - 1, W=512, k=64, causal=1,
                softmax_scale=1.25, dtype=1, flags=0)
    base.update(kw)
    return topo.TopoParams(**base)


@pytest.mark.parametrize("bad,code", [
    (dict(d=96), -2), (dict(dtype=7), -2), (dict(Hq=30), -1), (dict(n_ctx=0), -1), (dict(q_pos0=1 << 20), -1),
    (dict(W=-1), -1), (dict(k=4000, W=100), -1), (dict(softmax_scale=0.0), -1),
    (dict(softmax_scale=float("inf")), -1), (dict(causal=2), -1), (dict(flags=8), -1), (dict(n_q=2), -1),
])
def test_decode_rejects_bad_arguments_on_host(bad, code):
    lib = topo.load_library()
    p = _p(**bad)
    rc = lib.topo_attn_decode(ctypes.byref(p), None, None, None, None, None, None, None, 0, None)
    assert rc == code
    assert topo.topo_strerror(rc)


def test_decode_rejects_null_and_misaligned_pointers_and_small_workspace():
    lib = topo.load_library()
    p = _p()
    a = ctypes.c_void_p(1 << 40)  # never dereferenced: validation fails first
    mis = ctypes.c_void_p((1 << 40) + 8)
    assert lib.topo_attn_decode(ctypes.byref(p), a, None, a, a, None, None, a, 1 << 30, None) == -1
    assert lib.topo_attn_decode(ctypes.byref(p), mis, a, a, a, None, None, a, 1 << 30, None) == -1
    need = lib.topo_workspace_bytes(ctypes.byref(p), 0)
    assert need > 0
    assert lib.topo_attn_decode(ctypes.byref(p), a, a, a, a, None, None, a, need - 1, None) == -3
    assert lib.topo_select(ctypes.byref(p), a, a, None, None, a, need, None) == -1


def test_workspace_sizes():
    lib = topo.load_library()
    p = _p()
    dec = lib.topo_workspace_bytes(ctypes.byref(p), 0)
    assert 0 < dec < 64 << 20            # survivor lists of the 1M decode stay modest
    assert lib.topo_workspace_bytes(ctypes.byref(p), 3) > 0
    assert lib.topo_workspace_bytes(ctypes.byref(p), 9) == 0
    assert lib.topo_workspace_bytes(ctypes.byref(_p(d=96)), 0) == 0
    assert lib.topo_bw_probe(None, 16, None, None) == -1


def test_certified_decode_rejects_bad_arguments_on_host():
    lib = topo.load_library()
    a = ctypes.c_void_p(1 << 40)  # never dereferenced: validation fails first
    mis = ctypes.c_void_p((1 << 40) + 8)
    p = _p()
    need = lib.topo_workspace_bytes(ctypes.byref(p), 4)
    assert need >= lib.topo_workspace_bytes(ctypes.byref(p), 0) > 0
    # rho missing or misaligned, workspace too small
    assert lib.topo_attn_decode_certified(ctypes.byref(p), a, a, a, a, None, None, None, a, need, None) == -1
    assert lib.topo_attn_decode_certified(ctypes.byref(p), a, a, a, a, None, None, mis, a, need, None) == -1
    assert lib.topo_attn_decode_certified(ctypes.byref(p), a, a, a, a, None, None, a, a, need - 1, None) == -3
    # the dense fallback needs the dense scratch too, and is only accepted by the certified call
    pf = _p(flags=2)
    need_f = lib.topo_workspace_bytes(ctypes.byref(pf), 4)
    assert need_f > need
    assert lib.topo_attn_decode_certified(ctypes.byref(pf), a, a, a, a, None, None, a, a, need, None) == -3
    assert lib.topo_attn_decode(ctypes.byref(pf), a, a, a, a, None, None, a, 1 << 40, None) == -1
    assert lib.topo_attn_prefill(ctypes.byref(pf), a, a, a, a, None, None, a, 1 << 40, None) == -1
    assert lib.topo_attn_dense(ctypes.byref(pf), a, a, a, a, a, 1 << 40, None) == -1
    assert lib.topo_workspace_bytes(ctypes.byref(_p(n_q=2)), 4) == 0


def test_ragged_decode_and_kv_append_reject_bad_arguments_on_host():
    lib = topo.load_library()
    a = ctypes.c_void_p(1 << 40)  # never dereferenced: validation fails first
    mis8 = ctypes.c_void_p((1 << 40) + 4)
    p = _p()
    need = lib.topo_workspace_bytes(ctypes.byref(p), 5)
    # sized for a query at the cache's last row, whatever q_pos0 says
    assert need == lib.topo_workspace_bytes(ctypes.byref(_p(q_pos0=1000)), 5) == lib.topo_workspace_bytes(
        ctypes.byref(p), 0) > 0
    assert lib.topo_workspace_bytes(ctypes.byref(_p(causal=0)), 5) == 0
    assert lib.topo_workspace_bytes(ctypes.byref(_p(n_q=2)), 5) == 0
    # positions missing or misaligned, non-causal call, small workspace
    assert lib.topo_attn_decode_ragged(ctypes.byref(p), None, a, a, a, a, None, None, a, need, None) == -1
    assert lib.topo_attn_decode_ragged(ctypes.byref(p), mis8, a, a, a, a, None, None, a, need, None) == -1
    assert lib.topo_attn_decode_ragged(ctypes.byref(_p(causal=0)), a, a, a, a, a, None, None, a, need, None) == -1
    assert lib.topo_attn_decode_ragged(ctypes.byref(p), a, a, a, a, a, None, None, a, need - 1, None) == -3
    # append: every pointer required and aligned; shape checks as the other calls
    assert lib.topo_kv_append(ctypes.byref(p), None, a, a, a, a, None) == -1
    assert lib.topo_kv_append(ctypes.byref(p), mis8, a, a, a, a, None) == -1
    assert lib.topo_kv_append(ctypes.byref(p), a, None, a, a, a, None) == -1
    assert lib.topo_kv_append(ctypes.byref(p), a, a, a, ctypes.c_void_p((1 << 40) + 8), a, None) == -1
    assert lib.topo_kv_append(ctypes.byref(_p(d=96)), a, a, a, a, a, None) == -2


def test_noalloc_checks_on_host():
    """The allocation-free decode validates like topo_attn_decode and refuses, before any device
    call, a call whose workspace exceeds its static buffer."""
    lib = topo.load_library()
    a = ctypes.c_void_p(1 << 40)  # never dereferenced: validation fails first
    big = _p(B=8, n_ctx=1 << 22, q_pos0=(1 << 22) - 1)
    assert lib.topo_workspace_bytes(ctypes.byref(big), 0) > topo.TOPO_NOALLOC_MAX_BYTES
    assert lib.topo_attn_decode_noalloc(ctypes.byref(big), a, a, a, a, a, a, None) == -5
    assert topo.topo_strerror(-5)
    for bad, code in ((dict(d=96), -2), (dict(W=-1), -1), (dict(n_q=2), -1), (dict(flags=8), -1)):
        assert lib.topo_attn_decode_noalloc(ctypes.byref(_p(**bad)), a, a, a, a, a, a, None) == code


def _prefill_params(W, k, dtype=1):
    return topo.TopoParams(B=1, Hq=8, Hkv=8, d=128, n_ctx=8192, n_q=8192, q_pos0=0, W=W, k=k, causal=1,
                           softmax_scale=1.0, dtype=dtype, flags=0)


def test_prefill_set_size_limit_on_host():
    """The prefill's per-row finish keeps four rows in one block's LDS. With bf16 inputs and
    k <= 64 its compact layout does not grow with the set, so only TOPO_MAX_SET bounds 1 + W + k;
    otherwise the header's formula does (1871 at k = 64 for float32 inputs, 1849 at k = 96 for
    bf16). Larger sets are refused on the host, with a zero workspace size and TOPO_EUNSUPPORTED,
    before anything is launched."""
    lib = topo.load_library()
    ws = lambda W, k, dt=1: lib.topo_workspace_bytes(ctypes.byref(_prefill_params(W, k, dt)), 1)
    assert ws(4096 - 65, 64) > 0 and ws(2047, 64) > 0 and ws(2047, 8) > 0
    assert ws(1871 - 65, 64, 0) > 0 and ws(1872 - 65, 64, 0) == 0 and ws(2047, 64, 0) == 0
    assert ws(1849 - 97, 96) > 0 and ws(1850 - 97, 96) == 0
    # aligned host addresses stand in for device buffers: the size check refuses the call first
    buf = (ctypes.c_uint8 * 256)()
    a = (ctypes.addressof(buf) + 15) & ~15
    ptr = ctypes.c_void_p(a)
    for W, k, dt in ((1872 - 65, 64, 0), (2047, 64, 0), (1850 - 97, 96, 1)):
        prm = _prefill_params(W, k, dt)
        rc = lib.topo_attn_prefill(ctypes.byref(prm), ptr, ptr, ptr, ptr, ptr, ptr, ptr, ctypes.c_size_t(1 << 40), None)
        assert rc == -2, rc
        rc = lib.topo_select(ctypes.byref(prm), ptr, ptr, ptr, ptr, ptr, ctypes.c_size_t(1 << 40), None)
        assert rc == -2, rc


def test_library_shares_torchs_hip_runtime():
    """Loading the library before anything else imports torch still leaves one HIP runtime and
    one HSA runtime in the process (the binding imports torch first, whose runtime the library's
    dependency then resolves to); two runtimes would make torch's streams and allocations foreign
    to the library."""
    code = ("import os, dynamic_sparse_transformer_amd as t; t.load_library(); import torch; "
            "m = open(f'/proc/{os.getpid()}/maps').read().splitlines(); "
            "print(len({l.split()[-1] for l in m if 'libamdhip64' in l}), "
            "len({l.split()[-1] for l in m if 'libhsa-runtime64' in l}))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split()[-2:] == ["1", "1"], out.stdout
