"""GPU parity of the exactness certificate (topo_attn_decode_certified) with the oracle.

The certificate bounds the softmax mass a query's condensate set leaves out (the exactness claim
of "The Condensate Theorem: Transformers are O(n), Not O(n^2)", zh page, technical summary §2; hi
page, technical summary §2). The GPU bound is compared with oracle.certificate_bound (float64,
rounded up to float32 on the GPU); with the dense fallback, queries that are not certified get
dense attention, compared with oracle.dense_decode.
"""
import sys

import numpy as np
import pytest

import dynamic_sparse_transformer_amd as topo
import oracle
from tests._util import assert_out_close, assert_sets_equal, to_device, torch_cuda
from workloads import f32_to_bf16_bits, make_workload, bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_rho(rho_gpu, q, K, heads, W, k, scale, causal=True, q_pos=None):
    """rho from the GPU against the oracle's bound: never below it, at most a float32 rounding
    above it (both are float64 evaluations of the same expression, summed in different orders)."""
    n = K.shape[2]
    p = n - 1 if q_pos is None else q_pos
    Hq, Hkv = q.shape[1], K.shape[1]
    for b, h in heads:
        g = h // (Hq // Hkv)
        s = oracle.canonical_scores(q[b, h].reshape(-1), K[b, g])
        want = oracle.certificate_bound(s, p, W, k, float(np.float32(scale)), causal)
        got = float(rho_gpu[b, h])
        if want == 0.0 or np.isinf(want):
            assert got == want, (b, h, got, want)
        else:
            # at most one float32 step above (denormal steps included), never below
            hi = float(np.nextafter(np.float32(want * (1 + 1e-12)), np.float32(np.inf)))
            assert want * (1 - 1e-12) <= got <= hi, (b, h, got, want)


def peaky_and_flat(seed, n, d, dtype):
    """One kv head, four query heads: heads 0-1 point hard at planted keys (their sets carry
    nearly all the mass), heads 2-3 are nearly flat (most of the mass is left out)."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((1, 1, n, d), dtype=np.float32)
    V = rng.standard_normal((1, 1, n, d), dtype=np.float32)
    q = (0.05 * rng.standard_normal((1, 4, 1, d))).astype(np.float32)
    for h in (0, 1):
        j = int(rng.integers(10, n // 2))
        K[0, 0, j] = 12.0 * K[0, 0, j] / np.linalg.norm(K[0, 0, j])
        q[0, h, 0] = 40.0 * K[0, 0, j] / np.linalg.norm(K[0, 0, j])
    if dtype == "bf16":
        st = [f32_to_bf16_bits(x) for x in (q, K, V)]
        return [bf16_bits_to_f32(x) for x in st], st
    return [q, K, V], [q, K, V]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fallback", [False, True])
def test_certificate_and_dense_fallback(dtype, fallback):
    torch = torch_cuda()
    n, d, W, k, scale = 4096, 64, 32, 16, 0.125
    (q, K, V), store = peaky_and_flat(41, n, d, dtype)
    dq, dk, dv = (to_device(x, dtype) for x in store)
    out, sel, cnt, rho = topo.topo_attn_decode_certified(dq, dk, dv, W, k, scale, dense_fallback=fallback)
    torch.cuda.synchronize()
    out, sel, cnt, rho = out.cpu().numpy()[:, :, 0], sel.cpu().numpy()[:, :, 0], cnt.cpu().numpy()[:, :, 0], rho.cpu().numpy()
    heads = [(0, h) for h in range(4)]
    check_rho(rho, q, K, heads, W, k, scale)
    cert = rho < topo.TOPO_CERT_RHO
    assert cert[0, 0] and cert[0, 1] and not cert[0, 2] and not cert[0, 3]
    ro, rs, rc = oracle.topo_attn_decode(q, K, V, W, k, float(np.float32(scale)))
    assert_sets_equal(sel, cnt, rs, rc, "certified sets")
    dense = oracle.dense_decode(q, K, V, float(np.float32(scale)))
    for b, h in heads:
        want = dense[b, h] if (fallback and not cert[b, h]) else ro[b, h]
        assert_out_close(out[b, h], want, dtype, f"head {h} fallback={fallback}")


@pytest.mark.parametrize("cfg", [1, 2])
def test_certificate_small_configs(cfg):
    torch = torch_cuda()
    for over in ({}, {"beta": 16.0}):
        w = make_workload(cfg, **over)
        s = w.spec
        dq, dk, dv = (to_device(getattr(w, x), s.dtype) for x in ("q", "k", "v"))
        _, _, _, rho = topo.topo_attn_decode_certified(dq, dk, dv, s.W, s.k, float(s.softmax_scale))
        torch.cuda.synchronize()
        heads = [(0, h) for h in range(s.Hq)]
        check_rho(rho.cpu().numpy(), w.f32("q"), w.f32("k"), heads, s.W, s.k, float(s.softmax_scale))


@pytest.mark.parametrize("cfg,heads", [(4, [(0, 0), (2, 17), (3, 31)]), (5, [(0, 0), (0, 21)])])
def test_certificate_full_size(cfg, heads):
    """At 128K and 1M context (temperature 16) the sampled heads are certified, and their bound
    matches the oracle's."""
    torch = torch_cuda()
    w = make_workload(cfg)
    s = w.spec
    dq, dk, dv = (to_device(getattr(w, x), s.dtype) for x in ("q", "k", "v"))
    say(f"config {cfg}: certified decode")
    _, _, _, rho = topo.topo_attn_decode_certified(dq, dk, dv, s.W, s.k, float(s.softmax_scale))
    torch.cuda.synchronize()
    rho = rho.cpu().numpy()
    check_rho(rho, w.f32("q"), w.f32("k"), heads, s.W, s.k, float(s.softmax_scale))
    for b, h in heads:
        assert rho[b, h] < topo.TOPO_CERT_RHO
