"""GPU parity at the large-size edges: key-scan survivor lists merged before the finish (many
scan blocks per head), byte offsets past 4 GiB, and the prefill on both sides of its 2^31-byte
scan limit.

Method: "The Condensate Theorem: Transformers are O(n), Not O(n^2)", zh page, technical summary §3
(anchor, window and dynamic top-k; softmax over that set only).

At the sizes where the oracle cannot score every key in seconds, the keys are built so that the
top-k is known: background keys of small norm, and for each query head k planted keys along that
head's query with scores far above every background score (checked on the device in float32 with
torch before the call). The expected set is then {0} u planted u window, and the expected output
is the oracle's on the compacted problem that holds exactly those rows in position order (anchor
first, window last, k candidates, so every candidate is taken): the same softmax over the same
rows. Sets bit-exact; outputs within a relative 1e-2 (bf16 inputs).
"""
import sys

import numpy as np
import pytest

import dynamic_sparse_transformer_amd as topo
import oracle
from tests._util import assert_out_arith, assert_out_close, assert_sets_equal, to_device, torch_cuda
from tests.test_gpu_decode import random_case
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("ties", [False, True])
def test_decode_merged_survivor_lists(ties):
    """One kv head over about 1M keys: the scan runs hundreds of blocks for the head, so their
    survivor lists go through the merge kernel before the finish. Every head against the oracle."""
    torch = torch_cuda()
    B, Hq, Hkv, n, d, W, K = 1, 4, 1, 1_000_003, 128, 64, 64
    say("merged lists, ties", ties)
    vals, store = random_case(1700 + int(ties), B, Hq, Hkv, n, d, "bf16", ties=ties)
    dq, dk, dv = (to_device(x, "bf16") for x in store)
    scale = 1.0 / np.sqrt(d)
    out, sel, cnt = topo.topo_attn_decode(dq, dk, dv, W, K, scale)
    torch.cuda.synchronize()
    out, sel, cnt = out.cpu().numpy()[:, :, 0], sel.cpu().numpy()[:, :, 0], cnt.cpu().numpy()[:, :, 0]
    del dq, dk, dv
    torch.cuda.empty_cache()
    say("oracle")
    ro, rs, rc = oracle.topo_attn_decode(*vals, W, K, float(np.float32(scale)))
    assert_sets_equal(sel, cnt, rs, rc, f"merged ties={ties}")
    assert_out_close(out, ro, "bf16", f"merged ties={ties}")
    assert_out_arith(out, ro, f"merged ties={ties}")


def test_group_and_ragged_with_merged_lists():
    """The merge path under the shared selection (one set per kv head, G = 4) and under
    per-sequence positions (two sequences of one kv head each, at different lengths)."""
    torch = torch_cuda()
    B, Hq, Hkv, n, d, W, K = 2, 4, 1, 700_001, 128, 64, 32
    vals, store = random_case(1750, B, Hq, Hkv, n, d, "bf16")
    dq, dk, dv = (to_device(x, "bf16") for x in store)
    scale = 1.0 / np.sqrt(d)
    say("group selection over merged lists")
    out, sel, cnt = topo.topo_attn_decode(dq, dk, dv, W, K, scale, flags=topo.TOPO_FLAG_GROUP_SELECT)
    torch.cuda.synchronize()
    out, sel, cnt = out.cpu().numpy()[:, :, 0], sel.cpu().numpy()[:, :, 0], cnt.cpu().numpy()[:, :, 0]
    ro, rs, rc = oracle.topo_attn_decode_group(*vals, W, K, float(np.float32(scale)))
    assert_sets_equal(sel, cnt, rs, rc, "group merged")
    assert_out_close(out, ro, "bf16", "group merged")
    pos = [n - 1, 400_000]
    say("ragged positions over merged lists", pos)
    dpos = torch.tensor(pos, dtype=torch.int64, device="cuda")
    out, sel, cnt = topo.topo_attn_decode_ragged(dq, dk, dv, dpos, W, K, scale)
    torch.cuda.synchronize()
    out, sel, cnt = out.cpu().numpy()[:, :, 0], sel.cpu().numpy()[:, :, 0], cnt.cpu().numpy()[:, :, 0]
    del dq, dk, dv
    torch.cuda.empty_cache()
    q, k, v = vals
    for b, p in enumerate(pos):
        ro, rs, rc = oracle.topo_attn_decode(q[b:b + 1], k[b:b + 1, :, :p + 1], v[b:b + 1, :, :p + 1], W, K,
                                             float(np.float32(scale)))
        assert_sets_equal(sel[b:b + 1], cnt[b:b + 1], rs, rc, f"ragged merged b{b}")
        assert_out_close(out[b:b + 1], ro, "bf16", f"ragged merged b{b}")


def _device_cache(torch, n, d, seed, std):
    """(1, 1, n, d) bf16 cache of N(0, std^2) values, generated on the device in slices."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    x = torch.empty((1, 1, n, d), dtype=torch.bfloat16, device="cuda")
    step = 1 << 23
    for i in range(0, n, step):
        j = min(n, i + step)
        x[0, 0, i:j] = (torch.randn((j - i, d), generator=gen, device="cuda") * std).to(torch.bfloat16)
    return x


def _plant(torch, kc, q32, positions, rng):
    """Keys alpha * q_h / |q_h| (alpha in [2, 3)) at the given positions of head h's plant; returns
    the planted rows' float32 values as stored (bf16)."""
    rows = []
    for h, pos in enumerate(positions):
        u = q32[h] / np.linalg.norm(q32[h])
        alpha = 2.0 + rng.random(len(pos))
        rows.append((pos, bf16_bits_to_f32(f32_to_bf16_bits((alpha[:, None] * u[None, :]).astype(np.float32)))))
    for pos, r in rows:
        bits = f32_to_bf16_bits(r)
        kc[0, 0, torch.as_tensor(pos, device="cuda")] = to_device(bits, "bf16")
    return rows


def _check_planted_on_top(torch, kc, q32, positions, cand_hi, W):
    """Float32 device scores: every planted key of head h beats every other candidate of head h
    (positions 1 .. cand_hi) by a wide margin, so the top-k is the plant by construction."""
    n = kc.shape[2]
    for h, pos in enumerate(positions):
        qh = torch.as_tensor(q32[h], device="cuda")
        planted = torch.zeros(n, dtype=torch.bool, device="cuda")
        planted[torch.as_tensor(pos, device="cuda")] = True
        bg_max, pl_min = -np.inf, np.inf
        step = 1 << 23
        for i in range(0, n, step):
            j = min(n, i + step)
            s = kc[0, 0, i:j].float() @ qh
            idx = torch.arange(i, j, device="cuda")
            cand = (idx >= 1) & (idx <= cand_hi)
            pm = planted[i:j]
            if bool((cand & ~pm).any()):
                bg_max = max(bg_max, float(s[cand & ~pm].max()))
            if bool(pm.any()):
                pl_min = min(pl_min, float(s[pm].min()))
        assert pl_min > bg_max + 4.0, (h, pl_min, bg_max)


def _expected(positions_h, p, W):
    """The set of a query at position p whose top-k is the plant: {0} u plant u window, ascending."""
    w_lo = max(0, p - W + 1)
    return np.concatenate([[0], np.sort(np.asarray(positions_h)), np.arange(w_lo, p + 1)]).astype(np.int64)


def _gather_rows(torch, x, C):
    bits = x[0, 0, torch.as_tensor(C, device="cuda")].view(torch.int16).cpu().numpy().view(np.uint16)
    return bf16_bits_to_f32(bits)


def test_decode_beyond_4gib_offsets():
    """d = 64, 2^27 + 12,345 keys in one kv head: every K and V row past 16 GiB of its cache is
    addressed, key positions reach 2^27, and the survivor lists of 65K scan blocks are merged
    three times. Two query heads, each with 16 planted keys spread over the cache (the first
    and the last candidates among them)."""
    torch = torch_cuda()
    n, d, W, K, Hq = (1 << 27) + 12345, 64, 64, 16, 2
    say("decode beyond 4 GiB: generating", n, "keys")
    rng = np.random.default_rng(2701)
    q32 = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((Hq, d), dtype=np.float32)))
    kc = _device_cache(torch, n, d, 2702, 0.05)
    vc = _device_cache(torch, n, d, 2703, 1.0)
    p = n - 1
    cand_hi = p - W
    positions = []
    for h in range(Hq):
        pos = rng.choice(np.arange(3, cand_hi - 2, dtype=np.int64), size=K - 2, replace=False)
        positions.append(np.concatenate([pos, [1 + h, cand_hi - h]]).astype(np.int64))
    assert len(set(positions[0]) & set(positions[1])) == 0
    _plant(torch, kc, q32, positions, rng)
    _check_planted_on_top(torch, kc, q32, positions, cand_hi, W)
    dq = to_device(f32_to_bf16_bits(q32.reshape(1, Hq, 1, d)), "bf16")
    scale = 1.0 / np.sqrt(d)
    say("decode")
    out, sel, cnt = topo.topo_attn_decode(dq, kc, vc, W, K, scale)
    torch.cuda.synchronize()
    out, sel, cnt = out.cpu().numpy(), sel.cpu().numpy(), cnt.cpu().numpy()
    for h in range(Hq):
        C = _expected(positions[h], p, W)
        Kc, Vc = _gather_rows(torch, kc, C), _gather_rows(torch, vc, C)
        ro, rs, rc = oracle.topo_attn_decode(q32[None, h:h + 1, None, :], Kc[None, None], Vc[None, None], W, K,
                                             float(np.float32(scale)))
        assert cnt[0, h, 0] == len(C) and np.array_equal(sel[0, h, 0, :len(C)], C), f"set of head {h}"
        assert rc[0, 0] == len(C)
        assert_out_close(out[0, h, 0], ro[0, 0], "bf16", f"4GiB head {h}")
        assert_out_arith(out[0, h, 0], ro[0, 0], f"4GiB head {h}")
    del kc, vc, dq
    torch.cuda.empty_cache()


@pytest.mark.parametrize("side", ["below", "above"])
def test_prefill_at_the_scan_byte_limit(side):
    """Two query rows at the end of a cache whose key bytes are just below 2^31 (the matrix-core
    scan with its largest offsets) or just above (the exact per-row selection instead): d = 64,
    bf16, one head, 16 planted keys, W = 64."""
    torch = torch_cuda()
    d, W, K = 64, 64, 16
    n = (1 << 24) - 64 if side == "below" else (1 << 24) + 64
    say("prefill at the byte limit:", side, n)
    rng = np.random.default_rng(2801 + (side == "above"))
    q32 = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((2, d), dtype=np.float32)))
    kc = _device_cache(torch, n, d, 2802, 0.05)
    vc = _device_cache(torch, n, d, 2803, 1.0)
    # both rows score the plant of one direction: the mean of the two queries
    qm = q32.mean(axis=0, keepdims=True)
    p0 = n - 2
    cand_hi = p0 - W
    pos = np.concatenate([rng.choice(np.arange(2, cand_hi, dtype=np.int64), size=K - 2, replace=False),
                          [1, cand_hi]]).astype(np.int64)
    _plant(torch, kc, qm, [pos], rng)
    for i in range(2):  # row i's candidates are 1 .. p0 + i - W
        _check_planted_on_top(torch, kc, q32[i:i + 1], [pos], cand_hi + i, W)
    dq = to_device(f32_to_bf16_bits(q32.reshape(1, 1, 2, d)), "bf16")
    scale = 1.0 / np.sqrt(d)
    say("prefill")
    out, sel, cnt = topo.topo_attn_prefill(dq, kc, vc, W, K, scale, q_pos0=p0)
    torch.cuda.synchronize()
    out, sel, cnt = out.cpu().numpy(), sel.cpu().numpy(), cnt.cpu().numpy()
    for i in range(2):
        p = p0 + i
        C = _expected(pos, p, W)
        Kc, Vc = _gather_rows(torch, kc, C), _gather_rows(torch, vc, C)
        ro, rs, rc = oracle.topo_attn_decode(q32[None, i:i + 1, None, :], Kc[None, None], Vc[None, None], W, K,
                                             float(np.float32(scale)))
        assert cnt[0, 0, i] == len(C) and np.array_equal(sel[0, 0, i, :len(C)], C), f"set of row {i}"
        assert_out_close(out[0, 0, i], ro[0, 0], "bf16", f"prefill {side} row {i}")
        assert_out_arith(out[0, 0, i], ro[0, 0], f"prefill {side} row {i}")
    del kc, vc, dq
    torch.cuda.empty_cache()
