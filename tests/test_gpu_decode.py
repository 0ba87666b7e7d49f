"""GPU parity of the decode path (topo_attn_decode / topo_select / topo_attn_dense) with the CPU oracle.

Method: "The Condensate Theorem: Transformers are O(n), Not O(n^2)", zh page, technical summary §3
(condensate set) and fr page, technical summary §3 (softmax over the set). Index sets must match the
oracle bit for bit; outputs must meet |gpu - oracle| <= 1e-6 + 2e-6 |oracle| for float32 inputs and
a relative 1e-2 for bf16 inputs.
"""
import sys

import numpy as np
import pytest

import dynamic_sparse_transformer_amd as topo
import oracle
from tests._pool import pmap
from tests._util import (assert_out_arith, assert_out_close, assert_sets_equal, check_set_structure, to_device, torch_cuda)
from workloads import f32_to_bf16_bits, make_workload, spec

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_decode(q, k, v, W, K, scale, causal=True, q_pos=None, flags=0):
    out, sel, cnt = topo.topo_attn_decode(q, k, v, W, K, scale, causal=causal, q_pos0=q_pos, flags=flags)
    torch = torch_cuda()
    torch.cuda.synchronize()
    return out.cpu().numpy()[:, :, 0], sel.cpu().numpy()[:, :, 0], cnt.cpu().numpy()[:, :, 0]


def random_case(seed, B, Hq, Hkv, n, d, dtype, ties=False, equal=False):
    rng = np.random.default_rng(seed)
    if equal:
        q = np.ones((B, Hq, 1, d), np.float32)
        k = np.ones((B, Hkv, n, d), np.float32)
    elif ties:
        q = rng.integers(-2, 3, size=(B, Hq, 1, d)).astype(np.float32)
        k = rng.integers(-1, 2, size=(B, Hkv, n, d)).astype(np.float32)
    else:
        q = rng.standard_normal((B, Hq, 1, d), dtype=np.float32)
        k = rng.standard_normal((B, Hkv, n, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, n, d), dtype=np.float32)
    if dtype == "bf16":
        qs, ks, vs = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
        from workloads import bf16_bits_to_f32
        q, k, v = bf16_bits_to_f32(qs), bf16_bits_to_f32(ks), bf16_bits_to_f32(vs)
        return (q, k, v), (qs, ks, vs)
    return (q, k, v), (q, k, v)


def compare_case(vals, store, dtype, W, K, scale, causal=True, q_pos=None, flags=0, heads=None, what=""):
    q, k, v = vals
    dq, dk, dv = (to_device(x, dtype) for x in store)
    out, sel, cnt = run_decode(dq, dk, dv, W, K, scale, causal, q_pos, flags)
    ro, rs, rc = oracle.topo_attn_decode(q, k, v, W, K, float(np.float32(scale)), causal=causal, q_pos=q_pos,
                                         heads=heads)
    if heads is not None:
        idx = tuple(np.array(heads).T)
        assert_sets_equal(sel[idx], cnt[idx], rs[idx], rc[idx], what)
        assert_out_close(out[idx], ro[idx], dtype, what)
        if dtype == "bf16":
            assert_out_arith(out[idx], ro[idx], what)
    else:
        assert_sets_equal(sel, cnt, rs, rc, what)
        assert_out_close(out, ro, dtype, what)
        if dtype == "bf16":
            assert_out_arith(out, ro, what)
    return out, sel, cnt


@pytest.mark.parametrize("cfg", [1, 2])
def test_config_small_decode(cfg):
    torch_cuda()
    w = make_workload(cfg)
    s = w.spec
    say(f"config {cfg} {s.name}")
    compare_case((w.f32("q"), w.f32("k"), w.f32("v")), (w.q, w.k, w.v), s.dtype, s.W, s.k,
                 float(s.softmax_scale), what=s.name)


def test_config1_temperature_variant():
    torch_cuda()
    w = make_workload(1, beta=16.0)
    s = w.spec
    compare_case((w.f32("q"), w.f32("k"), w.f32("v")), (w.q, w.k, w.v), s.dtype, s.W, s.k,
                 float(s.softmax_scale), what="tiny beta=16")


CASES = [
    # (n, d, dtype, B, Hq, Hkv, W, K, causal, q_pos)
    (1, 64, "f32", 1, 1, 1, 4, 4, True, None),
    (2, 128, "bf16", 1, 2, 1, 0, 1, True, None),
    (63, 64, "f32", 2, 2, 2, 8, 8, True, None),
    (97, 64, "f32", 1, 1, 1, 64, 32, True, None),        # n = 1+W+k: every key
    (98, 64, "f32", 1, 1, 1, 64, 32, True, None),        # one candidate beyond the set
    (1000, 128, "bf16", 1, 4, 2, 16, 64, True, None),
    (1025, 64, "f32", 1, 3, 1, 0, 16, True, None),       # G = 3
    (4095, 128, "bf16", 2, 8, 2, 100, 7, True, None),
    (4097, 128, "bf16", 1, 8, 1, 31, 64, True, None),    # G = 8: two slices of 4
    (5000, 64, "bf16", 1, 4, 4, 128, 256, True, None),
    (9000, 128, "f32", 1, 2, 1, 256, 64, True, 6000),    # query in the middle of the cache
    (9000, 128, "bf16", 1, 4, 1, 64, 64, False, 4000),   # non-causal: keys after the query count
    (20000, 128, "bf16", 1, 4, 1, 512, 64, True, None),
    (33000, 64, "f32", 1, 2, 2, 0, 0, True, None),       # k = 0, W = 0: the anchor alone
    (3000, 128, "bf16", 1, 4, 2, 1000, 0, True, None),   # k = 0: sink + window
    (6000, 128, "f32", 1, 2, 1, 700, 16, True, None),     # window in 22 parts of 32 rows
    (70000, 128, "bf16", 1, 4, 1, 64, 1000, True, None),  # large k
]


@pytest.mark.parametrize("case", CASES, ids=[f"n{c[0]}-d{c[1]}-{c[2]}-G{c[4] // c[5]}-W{c[6]}-k{c[7]}"
                                            f"-{'c' if c[8] else 'nc'}" for c in CASES])
def test_decode_shapes_and_edges(case):
    torch_cuda()
    n, d, dtype, B, Hq, Hkv, W, K, causal, q_pos = case
    say("case", case)
    vals, store = random_case(100 + CASES.index(case), B, Hq, Hkv, n, d, dtype)
    compare_case(vals, store, dtype, W, K, 1.0 / np.sqrt(d), causal, q_pos, what=str(case))


@pytest.mark.parametrize("flags", [0, topo.TOPO_FLAG_EXACT_SELECT])
def test_decode_ties(flags):
    """Integer-valued keys: many equal scores, resolved to the lower position."""
    torch_cuda()
    vals, store = random_case(5, 1, 4, 2, 6000, 64, "f32", ties=True)
    compare_case(vals, store, "f32", 32, 48, 0.125, flags=flags, what="ties")


def test_decode_all_equal_keys():
    """Every score equal: the survivor lists overflow and the exact path must take the lowest
    positions."""
    torch_cuda()
    vals, store = random_case(6, 1, 2, 1, 20000, 128, "bf16", equal=True)
    out, sel, cnt = compare_case(vals, store, "bf16", 16, 32, 0.1, what="all equal")
    assert np.array_equal(sel[0, 0, 1:33], np.arange(1, 33))


def test_exact_flag_matches_fast_path():
    torch_cuda()
    vals, store = random_case(7, 1, 4, 1, 30000, 128, "bf16")
    dq, dk, dv = (to_device(x, "bf16") for x in store)
    a = run_decode(dq, dk, dv, 128, 64, 0.09)
    b = run_decode(dq, dk, dv, 128, 64, 0.09, flags=topo.TOPO_FLAG_EXACT_SELECT)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    assert_out_close(a[0], b[0], "f32", "fast vs exact")


def test_select_matches_decode_and_is_deterministic():
    torch = torch_cuda()
    vals, store = random_case(8, 2, 8, 2, 50000, 128, "bf16")
    dq, dk, dv = (to_device(x, "bf16") for x in store)
    a = run_decode(dq, dk, dv, 256, 64, 0.09)
    b = run_decode(dq, dk, dv, 256, 64, 0.09)
    sel, cnt = topo.topo_select(dq, dk, 256, 64, 0.09)
    torch.cuda.synchronize()
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(a[1], sel.cpu().numpy()[:, :, 0])
    assert np.array_equal(a[2], cnt.cpu().numpy()[:, :, 0])


def test_workspace_reuse_across_calls():
    torch = torch_cuda()
    vals1, store1 = random_case(9, 1, 4, 1, 40000, 128, "bf16")
    vals2, store2 = random_case(10, 1, 4, 1, 40000, 128, "bf16")
    d1 = [to_device(x, "bf16") for x in store1]
    d2 = [to_device(x, "bf16") for x in store2]
    nb = topo.topo_workspace_bytes(d1[0], d1[1], 64, 64, 0.09)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    o1 = topo.topo_attn_decode(*d1, 64, 64, 0.09, workspace=ws)
    o2 = topo.topo_attn_decode(*d2, 64, 64, 0.09, workspace=ws)
    torch.cuda.synchronize()
    r1 = oracle.topo_attn_decode(*vals1, 64, 64, float(np.float32(0.09)))
    r2 = oracle.topo_attn_decode(*vals2, 64, 64, float(np.float32(0.09)))
    assert np.array_equal(o1[1].cpu().numpy()[:, :, 0], r1[1])
    assert np.array_equal(o2[1].cpu().numpy()[:, :, 0], r2[1])


def test_invalid_arguments_write_nothing():
    torch = torch_cuda()
    q = torch.zeros((1, 2, 1, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 100, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full((1, 2, 1, 128), 7.0, device="cuda")
    with pytest.raises(topo.TopoError):
        topo.topo_attn_decode(q, k, k, 4000, 200, 0.1, out=out)        # 1+W+k above the cap
    with pytest.raises(topo.TopoError):
        topo.topo_attn_decode(q, k, k, 4, 4, -1.0, out=out)            # bad scale
    with pytest.raises(topo.TopoError):
        topo.topo_attn_decode(q, k, k, 4, 4, 0.1, q_pos0=100, out=out)  # query outside the cache
    with pytest.raises(topo.TopoError):
        topo.topo_attn_decode(q, k, k, 4, 4, 0.1, out=out, workspace=torch.empty(8, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def _full_config(cfg, sample_heads):
    torch = torch_cuda()
    say(f"config {cfg}: generating")
    w = make_workload(cfg)
    s = w.spec
    dq, dk, dv = (to_device(getattr(w, x), s.dtype) for x in ("q", "k", "v"))
    say(f"config {cfg}: decode on GPU")
    out, sel, cnt = run_decode(dq, dk, dv, s.W, s.k, float(s.softmax_scale))
    del dq, dk, dv
    torch.cuda.empty_cache()
    check_set_structure(sel, cnt, s.n_ctx - 1, s.W, s.k, s.n_ctx - 1 - s.W)
    say(f"config {cfg}: oracle on {len(sample_heads)} heads")
    ro, rs, rc = oracle.topo_attn_decode(w.f32("q"), w.f32("k"), w.f32("v"), s.W, s.k, float(s.softmax_scale),
                                         heads=sample_heads)
    idx = tuple(np.array(sample_heads).T)
    assert_sets_equal(sel[idx], cnt[idx], rs[idx], rc[idx], s.name)
    assert_out_close(out[idx], ro[idx], s.dtype, s.name)
    if s.dtype == "bf16":
        assert_out_arith(out[idx], ro[idx], s.name)
    # planted keys are retrieved (synthetic needle retrieval)
    hits = [np.isin(w.planted[(b, h)], sel[b, h]).mean() for (b, h) in w.planted]
    say(f"config {cfg}: planted recall {np.mean(hits):.4f}")
    assert np.mean(hits) > 0.99


@pytest.mark.parametrize("ties", [False, True])
def test_multi_run_scan_blocks(ties):
    """32 (batch, kv head) groups over 64K keys: enough blocks that each key-scan block ranks more
    than one run of keys (and, with many equal scores, cuts its list between runs)."""
    torch_cuda()
    vals, store = random_case(900 + int(ties), 4, 32, 8, 65536, 128, "bf16", ties=ties)
    heads = [(0, 0), (1, 7), (2, 16), (3, 31), (3, 2)]
    compare_case(vals, store, "bf16", 64, 64, 0.088, heads=heads, what=f"multi-run ties={ties}")


@pytest.mark.parametrize("cfg,n_ctx", [(2, None), (5, 65536), (5, None)])
def test_dense_pillar_matches_oracle(cfg, n_ctx):
    """The dense pillar layer (zh page, technical summary §3), at the 1M-token decode's full size
    too (the pillar comparison that configuration asks for): four query heads, one per two kv heads."""
    torch_cuda()
    over = {} if n_ctx is None else {"n_ctx": n_ctx}
    w = make_workload(cfg, **over)
    s = w.spec
    dq, dk, dv = (to_device(getattr(w, x), s.dtype) for x in ("q", "k", "v"))
    say(f"dense pillar {s.name} n={s.n_ctx} on GPU")
    out = topo.topo_attn_dense(dq, dk, dv, float(s.softmax_scale)).cpu().numpy()[:, :, 0]
    del dq, dk, dv
    heads = [(0, h) for h in range(0, s.Hq, max(1, s.Hq // 4))]
    q, k, v = w.f32("q"), w.f32("k"), w.f32("v")
    say(f"dense pillar: oracle on {len(heads)} heads")
    parts = pmap(lambda bh: oracle.dense_decode(q, k, v, float(s.softmax_scale), heads=[bh])[bh], heads)
    ref = np.full_like(out, np.nan)
    for bh, o in zip(heads, parts):
        ref[bh] = o
    idx = tuple(np.array(heads).T)
    assert_out_close(out[idx], ref[idx], s.dtype, f"dense {s.name}")
