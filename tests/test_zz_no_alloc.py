"""The allocation-free decode entry point, topo_attn_decode_noalloc, against topo_attn_decode.

It runs the same kernels as topo_attn_decode (the condensate-set attention of "The Condensate
Theorem: Transformers are O(n), Not O(n^2)", zh page, technical summary §3; fr page, technical
summary §3) with its workspace in the library's static per-GPU buffer. Two calls in a row, the
second smaller than the first, each compared with topo_attn_decode on the same inputs: index sets
bit for bit, outputs within 1e-6 + 2e-6 |ref| (float32 inputs) or a relative 1e-2 (bf16 inputs).
"""
import ctypes
import sys

import numpy as np
import pytest

import dynamic_sparse_transformer_amd as topo
from tests._util import assert_out_close, assert_sets_equal, to_device, torch_cuda
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def inputs(seed, B, Hq, Hkv, n, d, dtype):
    rng = np.random.default_rng(seed)
    arrs = [rng.standard_normal(s, dtype=np.float32) for s in ((B, Hq, 1, d), (B, Hkv, n, d), (B, Hkv, n, d))]
    if dtype == "bf16":
        arrs = [f32_to_bf16_bits(a) for a in arrs]
    return [to_device(a, dtype) for a in arrs]


def compare(seed, B, Hq, Hkv, n, d, dtype, W, K, scale):
    torch = torch_cuda()
    say(f"no-alloc case seed {seed}: B{B} Hq{Hq} Hkv{Hkv} n{n} d{d} {dtype} W{W} k{K}")
    q, k, v = inputs(seed, B, Hq, Hkv, n, d, dtype)
    need = topo.topo_workspace_bytes(q, k, W, K, scale)
    assert 0 < need <= topo.TOPO_NOALLOC_MAX_BYTES
    o1, s1, c1 = topo.topo_attn_decode_noalloc(q, k, v, W, K, scale)
    o2, s2, c2 = topo.topo_attn_decode(q, k, v, W, K, scale)
    torch.cuda.synchronize()
    o1, s1, c1 = o1.cpu().numpy(), s1.cpu().numpy(), c1.cpu().numpy()
    o2, s2, c2 = o2.cpu().numpy(), s2.cpu().numpy(), c2.cpu().numpy()
    assert_sets_equal(s1, c1, s2, c2, f"no-alloc seed {seed}")
    assert_out_close(o1, o2, dtype, f"no-alloc seed {seed}")
    say(f"  workspace {need} bytes, sets equal, outputs bitwise equal: {np.array_equal(o1, o2)}")


def test_noalloc_matches_decode_twice_second_smaller():
    compare(8101, 1, 32, 8, 262144, 128, "bf16", 256, 64, 16.0 / np.sqrt(128))
    compare(8102, 2, 4, 2, 5000, 64, "f32", 32, 16, 0.125)


def test_noalloc_rejects_oversize_without_launch():
    torch = torch_cuda()
    lib = topo.load_library()
    p = topo.TopoParams(8, 32, 8, 128, 1 << 22, 1, (1 << 22) - 1, 512, 64, 1, 0.1, 1, 0)
    assert lib.topo_workspace_bytes(ctypes.byref(p), 0) > topo.TOPO_NOALLOC_MAX_BYTES
    a = ctypes.c_void_p(1 << 40)  # never dereferenced: the size check fails first
    assert lib.topo_attn_decode_noalloc(ctypes.byref(p), a, a, a, a, a, a, None) == -5
