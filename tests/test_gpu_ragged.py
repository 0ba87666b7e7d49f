"""GPU parity of the decode loop: per-sequence positions (topo_attn_decode_ragged) and the KV-cache
append (topo_kv_append), against the CPU oracle.

Method: "The Condensate Theorem: Transformers are O(n), Not O(n^2)", zh page, technical summary §3
(the set is chosen again at every generated token); fr page, technical summary §3 (softmax over the
set). Sets bit-exact; outputs within 1e-6 + 2e-6 |ref| (float32 inputs) or a relative 1e-2 (bf16).
"""
import sys

import numpy as np
import pytest

import dynamic_sparse_transformer_amd as topo
import oracle
from tests._util import assert_out_arith, assert_out_close, assert_sets_equal, to_device, torch_cuda
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_case(seed, B, Hq, Hkv, n, d, dtype):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, 1, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, n, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, n, d), dtype=np.float32)
    if dtype == "bf16":
        st = tuple(f32_to_bf16_bits(x) for x in (q, k, v))
        return tuple(bf16_bits_to_f32(x) for x in st), st
    return (q, k, v), (q, k, v)


def check_against_oracle(vals, pos, out, sel, cnt, W, K, scale, dtype, what):
    q, k, v = vals
    for b, p in enumerate(pos):
        o_ref, s_ref, c_ref = oracle.topo_attn_decode(q[b:b + 1], k[b:b + 1], v[b:b + 1], W, K, scale, True, q_pos=int(p))
        for h in range(q.shape[1]):
            assert_sets_equal(sel[b, h], cnt[b, h], s_ref[0, h], c_ref[0, h], f"{what} b{b} p{p} h{h}")
            assert_out_close(out[b, h], o_ref[0, h], dtype, f"{what} b{b} p{p} h{h}")
            if dtype == "bf16":
                assert_out_arith(out[b, h], o_ref[0, h], f"{what} b{b} p{p} h{h}")


# (seed, B, Hq, Hkv, n, d, dtype, positions, W, k): positions cover the full cache, a mid-length
# sequence, one with at most k candidates (all taken) and one inside the window (no candidates)
CASES = [
    (11, 4, 4, 2, 3000, 128, "bf16", [2999, 1234, 40, 10], 32, 16),
    (12, 4, 4, 1, 2100, 64, "f32", [150, 2099, 1, 777], 64, 32),
    (13, 2, 8, 8, 5000, 128, "bf16", [4999, 2500], 128, 64),
    # a window wider than most sequences: parts of the window past a short sequence stay empty
    (14, 3, 4, 2, 3000, 128, "f32", [2999, 300, 5], 700, 16),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[1]}-n{c[4]}-d{c[5]}-{c[6]}-W{c[8]}-k{c[9]}" for c in CASES])
def test_ragged_decode_matches_oracle_and_plain_calls(case):
    torch = torch_cuda()
    seed, B, Hq, Hkv, n, d, dtype, pos, W, K = case
    say("case", case)
    vals, store = make_case(seed, B, Hq, Hkv, n, d, dtype)
    dq, dk, dv = (to_device(x, dtype) for x in store)
    scale = 1.0 / np.sqrt(d)
    dpos = torch.tensor(pos, dtype=torch.int64, device="cuda")
    out, sel, cnt = topo.topo_attn_decode_ragged(dq, dk, dv, dpos, W, K, scale)
    torch.cuda.synchronize()
    out, sel, cnt = out.cpu().numpy()[:, :, 0], sel.cpu().numpy()[:, :, 0], cnt.cpu().numpy()[:, :, 0]
    check_against_oracle(vals, pos, out, sel, cnt, W, K, scale, dtype, "ragged")
    # each sequence alone through the one-position call: the same sets and outputs
    for b, p in enumerate(pos):
        o1, s1, c1 = topo.topo_attn_decode(dq[b:b + 1], dk[b:b + 1], dv[b:b + 1], W, K, scale, q_pos0=p)
        torch.cuda.synchronize()
        assert np.array_equal(s1.cpu().numpy()[0, :, 0], sel[b]) and np.array_equal(c1.cpu().numpy()[0, :, 0], cnt[b])
        assert np.allclose(o1.cpu().numpy()[0, :, 0], out[b], rtol=1e-6, atol=1e-7)


def test_kv_append_writes_only_the_given_rows():
    torch = torch_cuda()
    B, Hkv, n, d = 3, 2, 64, 128
    rng = np.random.default_rng(5)
    kc = torch.tensor(rng.standard_normal((B, Hkv, n, d), dtype=np.float32), device="cuda").to(torch.bfloat16)
    vc = torch.tensor(rng.standard_normal((B, Hkv, n, d), dtype=np.float32), device="cuda").to(torch.bfloat16)
    k0, v0 = kc.clone(), vc.clone()
    kn = torch.tensor(rng.standard_normal((B, Hkv, d), dtype=np.float32), device="cuda").to(torch.bfloat16)
    vn = torch.tensor(rng.standard_normal((B, Hkv, d), dtype=np.float32), device="cuda").to(torch.bfloat16)
    pos = torch.tensor([5, n - 1, n], dtype=torch.int64, device="cuda")  # the last one is outside the cache
    topo.topo_kv_append(kc, vc, kn, vn, pos)
    torch.cuda.synchronize()
    want_k, want_v = k0.clone(), v0.clone()
    want_k[0, :, 5] = kn[0]
    want_v[0, :, 5] = vn[0]
    want_k[1, :, n - 1] = kn[1]
    want_v[1, :, n - 1] = vn[1]
    assert torch.equal(kc, want_k) and torch.equal(vc, want_v)


def test_decode_loop_append_then_attend():
    """Four generated tokens for three sequences of different lengths: append the token's k, v at
    pos[b], attend at pos[b], advance pos on the device; every step against the oracle on the
    grown caches."""
    torch = torch_cuda()
    B, Hq, Hkv, n, d, W, K = 3, 4, 2, 1200, 128, 24, 16
    vals, store = make_case(21, B, Hq, Hkv, n, d, "bf16")
    q0, kf, vf = (x.copy() for x in vals)
    dk, dv = to_device(store[1], "bf16"), to_device(store[2], "bf16")
    pos0 = [900, 400, 30]
    dpos = torch.tensor(pos0, dtype=torch.int64, device="cuda")
    rng = np.random.default_rng(22)
    scale = 1.0 / np.sqrt(d)
    for step in range(4):
        qs = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((B, Hq, 1, d), dtype=np.float32)))
        kn = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((B, Hkv, d), dtype=np.float32)))
        vn = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((B, Hkv, d), dtype=np.float32)))
        pos = [p + step for p in pos0]
        for b in range(B):
            kf[b, :, pos[b]] = kn[b]
            vf[b, :, pos[b]] = vn[b]
        topo.topo_kv_append(dk, dv, to_device(f32_to_bf16_bits(kn), "bf16"), to_device(f32_to_bf16_bits(vn), "bf16"), dpos)
        out, sel, cnt = topo.topo_attn_decode_ragged(to_device(f32_to_bf16_bits(qs), "bf16"), dk, dv, dpos, W, K, scale)
        dpos += 1
        torch.cuda.synchronize()
        say("step", step, "positions", pos)
        check_against_oracle((qs, kf, vf), pos, out.cpu().numpy()[:, :, 0], sel.cpu().numpy()[:, :, 0],
                             cnt.cpu().numpy()[:, :, 0], W, K, scale, "bf16", f"step {step}")


def test_decode_loop_step_in_a_graph():
    """Append, ragged decode and position advance captured once into a HIP graph; every replay
    (one generated token) equals the same step run eagerly on a copy of the state."""
    torch = torch_cuda()
    B, Hq, Hkv, n, d, W, K = 2, 8, 2, 4096, 128, 64, 32
    vals, store = make_case(31, B, Hq, Hkv, n, d, "bf16")
    dq, dk, dv = (to_device(x, "bf16") for x in store)
    scale = 1.0 / np.sqrt(d)
    rng = np.random.default_rng(32)
    kn = to_device(f32_to_bf16_bits(rng.standard_normal((B, Hkv, d), dtype=np.float32)), "bf16")
    vn = to_device(f32_to_bf16_bits(rng.standard_normal((B, Hkv, d), dtype=np.float32)), "bf16")
    pos = torch.tensor([3000, 1000], dtype=torch.int64, device="cuda")
    ws = torch.empty(topo.topo_workspace_bytes(dq, dk, W, K, scale, op=topo.TOPO_OP_DECODE_RAGGED),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, 1, d), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, Hq, 1, 1 + W + K), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, Hq, 1), dtype=torch.int32, device="cuda")
    # eager reference on copies of the caches and positions
    rk, rv, rpos = dk.clone(), dv.clone(), pos.clone()
    ref = []
    for _ in range(3):
        topo.topo_kv_append(rk, rv, kn, vn, rpos)
        o, s, c = topo.topo_attn_decode_ragged(dq, rk, rv, rpos, W, K, scale)
        rpos += 1
        torch.cuda.synchronize()
        ref.append((o.cpu().clone(), s.cpu().clone(), c.cpu().clone()))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        topo.topo_kv_append(dk, dv, kn, vn, pos, stream=stream)
        topo.topo_attn_decode_ragged(dq, dk, dv, pos, W, K, scale, out=out, sel_idx=sel, sel_count=cnt,
                                     workspace=ws, stream=stream)
        pos.add_(1)
    torch.cuda.synchronize()
    for step in range(3):
        graph.replay()
        torch.cuda.synchronize()
        o, s, c = ref[step]
        assert torch.equal(sel.cpu(), s) and torch.equal(cnt.cpu(), c), f"replay {step}"
        assert torch.allclose(out.cpu(), o, rtol=1e-6, atol=1e-7), f"replay {step}"
    assert pos.cpu().tolist() == [3003, 1003]


def test_ragged_at_the_128k_gqa_workload():
    """The batch-4 GQA workload at full size (128K-row caches), each sequence at its own position:
    sampled heads of every sequence against the oracle on that sequence's prefix."""
    from workloads import make_workload
    torch = torch_cuda()
    w = make_workload(4)
    s = w.spec
    dq, dk, dv = (to_device(getattr(w, x), s.dtype) for x in ("q", "k", "v"))
    pos = [s.n_ctx - 1, 100000, 65536, 3000]
    dpos = torch.tensor(pos, dtype=torch.int64, device="cuda")
    say("128K ragged decode on GPU, positions", pos)
    out, sel, cnt = topo.topo_attn_decode_ragged(dq, dk, dv, dpos, s.W, s.k, float(s.softmax_scale))
    torch.cuda.synchronize()
    out, sel, cnt = out.cpu().numpy()[:, :, 0], sel.cpu().numpy()[:, :, 0], cnt.cpu().numpy()[:, :, 0]
    q, k, v = w.f32("q"), w.f32("k"), w.f32("v")
    for b, p in enumerate(pos):
        heads = [(0, h) for h in (b, 9 + b, 31 - b)]
        say(f"oracle b{b} p{p}")
        o_ref, s_ref, c_ref = oracle.topo_attn_decode(q[b:b + 1], k[b:b + 1, :, :p + 1], v[b:b + 1, :, :p + 1], s.W, s.k,
                                                      float(s.softmax_scale), True, heads=heads)
        for _, h in heads:
            assert_sets_equal(sel[b, h], cnt[b, h], s_ref[0, h], c_ref[0, h], f"128K b{b} p{p} h{h}")
            assert_out_close(out[b, h], o_ref[0, h], s.dtype, f"128K b{b} p{p} h{h}")
