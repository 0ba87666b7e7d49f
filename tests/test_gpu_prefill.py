"""GPU parity of the many-query (prefill) path, topo_attn_prefill / topo_select, with the CPU oracle.

Method: "The Condensate Theorem: Transformers are O(n), Not O(n^2)", zh page, technical summary §3
(every query position i attends to its own condensate set C_i); fr page, technical summary §3
(softmax over C_i). Index sets bit-exact; outputs within 1e-6 + 2e-6|ref| (float32 inputs) or a
relative 1e-2 (bf16 inputs).
"""
import sys

import numpy as np
import pytest

import dynamic_sparse_transformer_amd as topo
import oracle
from tests._util import assert_out_arith, assert_out_close, assert_sets_equal, to_device, torch_cuda
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_prefill(q, k, v, W, K, scale, causal=True, q_pos0=0, flags=0):
    torch = torch_cuda()
    out, sel, cnt = topo.topo_attn_prefill(q, k, v, W, K, scale, causal=causal, q_pos0=q_pos0, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy(), sel.cpu().numpy(), cnt.cpu().numpy()


def compare_rows(vals, out, sel, cnt, rows, W, K, scale, causal, q_pos0, dtype, what):
    Q, Kc, V = vals  # (B, Hq, n_q, d), (B, Hkv, n, d)
    S = 1 + W + K
    for b in range(Q.shape[0]):
        res = oracle.topo_attn_rows(Q[b], Kc[b], V[b], rows, W, K, float(np.float32(scale)), causal, q_pos0)
        for (h, i), (o, C) in res.items():
            ref_sel = np.full(S, -1, np.int32)
            ref_sel[:C.size] = C
            assert_sets_equal(sel[b, h, i], np.int32(cnt[b, h, i]), ref_sel, np.int32(C.size), f"{what} b{b} h{h} i{i}")
            assert_out_close(out[b, h, i], o, dtype, f"{what} b{b} h{h} i{i}")
            if dtype == "bf16":
                assert_out_arith(out[b, h, i], o, f"{what} b{b} h{h} i{i}")


def random_prefill(seed, B, Hq, Hkv, n, n_q, d, dtype, ties=False):
    rng = np.random.default_rng(seed)
    if ties:
        q = rng.integers(-2, 3, size=(B, Hq, n_q, d)).astype(np.float32)
        k = rng.integers(-1, 2, size=(B, Hkv, n, d)).astype(np.float32)
    else:
        q = rng.standard_normal((B, Hq, n_q, d), dtype=np.float32)
        k = rng.standard_normal((B, Hkv, n, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, n, d), dtype=np.float32)
    if dtype == "bf16":
        st = tuple(f32_to_bf16_bits(x) for x in (q, k, v))
        return tuple(bf16_bits_to_f32(x) for x in st), st
    return (q, k, v), (q, k, v)


def sample_rows(rng, Hq, n_q, q_pos0, W, K, extra=12):
    base = {0, 1, n_q - 1, n_q // 2}
    for p in (W - 1, W, W + 1, W + K, W + K + 1, W + K + 2):
        if 0 <= p - q_pos0 < n_q:
            base.add(p - q_pos0)
    rows = set()
    for h in range(Hq):
        for i in base:
            if 0 <= i < n_q:
                rows.add((h, i))
        for i in rng.integers(0, n_q, size=extra):
            rows.add((h, int(i)))
    return sorted(rows)


CASES = [
    # (n, n_q, q_pos0, d, dtype, B, Hq, Hkv, W, K, causal)
    (300, 300, 0, 128, "bf16", 1, 2, 1, 16, 8, True),
    (1000, 1000, 0, 128, "bf16", 1, 4, 2, 64, 32, True),
    (2049, 2049, 0, 64, "bf16", 2, 2, 2, 128, 64, True),
    (3000, 700, 2300, 128, "bf16", 1, 2, 1, 100, 96, True),   # chunked prefill: the last 700 queries
    (1500, 1500, 0, 128, "bf16", 1, 2, 1, 0, 40, True),       # no window
    (1500, 1500, 0, 128, "bf16", 1, 2, 1, 50, 0, True),       # sink + window only
    (900, 300, 200, 128, "bf16", 1, 2, 1, 32, 16, False),     # non-causal
    (700, 700, 0, 64, "f32", 1, 2, 1, 32, 16, True),          # float32: exact selection path
    (1200, 1200, 0, 128, "bf16", 1, 2, 1, 40, 150, True),     # k above the MFMA scan's limit
    (2500, 2500, 0, 128, "bf16", 1, 1, 1, 2047, 64, True),    # bf16, k <= 64: a set past the general layout's limit
    (2500, 2500, 0, 128, "bf16", 1, 1, 1, 1752, 96, True),    # bf16, k = 96: the largest set (1 + W + k = 1849)
    (2000, 2000, 0, 64, "f32", 1, 1, 1, 1806, 64, True),      # float32: the largest set at k = 64 (1871)
    # more scan jobs than the GPU holds at once: each block takes several in snake order
    (16384, 16384, 0, 128, "bf16", 1, 12, 4, 128, 64, True),  # 1536 jobs, one list (12 heads)
    (8192, 8192, 0, 64, "bf16", 2, 20, 4, 64, 32, True),      # 2560 jobs, eight lists of 5 heads
]


@pytest.mark.parametrize("case", CASES, ids=[f"n{c[0]}-q{c[1]}@{c[2]}-d{c[3]}-{c[4]}-G{c[6] // c[7]}-W{c[8]}-k{c[9]}"
                                            f"-{'c' if c[10] else 'nc'}" for c in CASES])
def test_prefill_shapes_and_edges(case):
    torch_cuda()
    n, n_q, q_pos0, d, dtype, B, Hq, Hkv, W, K, causal = case
    say("case", case)
    vals, store = random_prefill(200 + CASES.index(case), B, Hq, Hkv, n, n_q, d, dtype)
    dq, dk, dv = (to_device(x, dtype) for x in store)
    scale = 1.0 / np.sqrt(d)
    out, sel, cnt = run_prefill(dq, dk, dv, W, K, scale, causal, q_pos0)
    rows = sample_rows(np.random.default_rng(1), Hq, n_q, q_pos0, W, K)
    compare_rows(vals, out, sel, cnt, rows, W, K, scale, causal, q_pos0, dtype, str(case))


def test_prefill_ties_and_exact_flag():
    torch_cuda()
    vals, store = random_prefill(7, 1, 2, 1, 1600, 1600, 64, "bf16", ties=True)
    dq, dk, dv = (to_device(x, "bf16") for x in store)
    rows = sample_rows(np.random.default_rng(2), 2, 1600, 0, 32, 48)
    a = run_prefill(dq, dk, dv, 32, 48, 0.125)
    compare_rows(vals, *a, rows, 32, 48, 0.125, True, 0, "bf16", "ties")
    b = run_prefill(dq, dk, dv, 32, 48, 0.125, flags=topo.TOPO_FLAG_EXACT_SELECT)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


def test_prefill_select_matches_attn():
    torch = torch_cuda()
    vals, store = random_prefill(8, 1, 4, 2, 2500, 2500, 128, "bf16")
    dq, dk, dv = (to_device(x, "bf16") for x in store)
    o, s1, c1 = run_prefill(dq, dk, dv, 64, 64, 0.09)
    s2, c2 = topo.topo_select(dq, dk, 64, 64, 0.09, q_pos0=0)
    torch.cuda.synchronize()
    assert np.array_equal(s1, s2.cpu().numpy()) and np.array_equal(c1, c2.cpu().numpy())
