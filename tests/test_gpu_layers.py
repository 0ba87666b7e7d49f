"""GPU parity of a decode step through a stack of attention layers (topo_attn_decode_layers) with
the CPU oracle: pillar layers dense, the others with their own (W, k) (zh page, technical summary
§3). Sets bit-exact; outputs within 1e-6 + 2e-6 |ref| (float32) or a relative 1e-2 (bf16)."""
import sys

import numpy as np
import pytest

import dynamic_sparse_transformer_amd as topo
import oracle
from tests._util import assert_out_close, assert_sets_equal, to_device, torch_cuda
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("L,n,d,dtype", [(8, 1500, 64, "f32"), (32, 700, 128, "bf16")])
def test_layer_stack_matches_oracle(L, n, d, dtype):
    torch_cuda()
    B, Hq, Hkv = 2, 4, 2
    rng = np.random.default_rng(100 + L)
    plan = topo.pillar_schedule(L, 256, 64, 32, 8)
    scale = 1.0 / np.sqrt(d)
    vals, dev = [], []
    for _ in range(L):
        x = [rng.standard_normal(s, dtype=np.float32) for s in ((B, Hq, 1, d), (B, Hkv, n, d), (B, Hkv, n, d))]
        if dtype == "bf16":
            bits = [f32_to_bf16_bits(a) for a in x]
            x = [bf16_bits_to_f32(b) for b in bits]
            dev.append(tuple(to_device(b, "bf16") for b in bits))
        else:
            dev.append(tuple(to_device(a, "f32") for a in x))
        vals.append(x)
    say(f"stack of {L} layers, pillars at", [i for i, (p, _, _) in enumerate(plan) if p])
    res = topo.topo_attn_decode_layers(dev, plan, scale)
    torch_cuda().cuda.synchronize()
    for i, ((q, k, v), (pillar, W, kk), (out, sel, cnt)) in enumerate(zip(vals, plan, res)):
        o = out.cpu().numpy()[:, :, 0]
        if pillar:
            assert sel is None
            ref = oracle.dense_decode(q, k, v, scale)
            assert_out_close(o, ref, dtype, f"layer {i} (pillar)")
        else:
            o_ref, s_ref, c_ref = oracle.topo_attn_decode(q, k, v, W, kk, scale)
            assert_sets_equal(sel.cpu().numpy()[:, :, 0], cnt.cpu().numpy()[:, :, 0], s_ref, c_ref, f"layer {i}")
            assert_out_close(o, o_ref, dtype, f"layer {i}")
