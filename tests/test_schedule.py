"""Host logic of the layer stack: the pillar / layer-adaptive plan (zh page, technical summary §3:
about one dense "pillar" layer in sixteen; wider windows in early layers, leaner sets in later
ones) and the C ABI's checks of a layer list (no GPU needed: validation fails before any launch)."""
import ctypes

import pytest

import dynamic_sparse_transformer_amd as topo


@pytest.mark.parametrize("L", [1, 2, 8, 15, 16, 24, 32, 40, 48, 64, 80])
def test_pillar_schedule_shape(L):
    plan = topo.pillar_schedule(L, 512, 64, 128, 16)
    assert len(plan) == L
    pillars = [i for i, (p, _, _) in enumerate(plan) if p]
    assert len(pillars) == max(1, round(L / 16))
    assert pillars[0] == 0
    gaps = {b - a for a, b in zip(pillars, pillars[1:])}
    assert all(abs(g - L / len(pillars)) < 1 for g in gaps)  # evenly spaced
    W = [w for _, w, _ in plan]
    k = [kk for _, _, kk in plan]
    assert W[0] == 512 and k[0] == 64
    if L > 1:
        assert W[-1] == 128 and k[-1] == 16
    assert all(a >= b for a, b in zip(W, W[1:])) and all(a >= b for a, b in zip(k, k[1:]))


def test_pillar_schedule_constant_sizes():
    assert {(w, k) for _, w, k in topo.pillar_schedule(32, 256, 64)} == {(256, 64)}


def _p(**kw):
    base = dict(B=1, Hq=32, Hkv=8, d=128, n_ctx=1 << 17, n_q=1, q_pos0=(1 << 17) - 1, W=0, k=0, causal=1,
                softmax_scale=1.25, dtype=1, flags=0)
    base.update(kw)
    return topo.TopoParams(**base)


def _layers(plan, ptr=1 << 40):
    arr = (topo.TopoLayer * len(plan))()
    for i, (pillar, W, k) in enumerate(plan):
        arr[i] = topo.TopoLayer(ptr, ptr, ptr, ptr, None, None, W, k, int(pillar), 0)
    return arr


def test_layer_list_checks_before_launch():
    lib = topo.load_library()
    p = _p()
    plan = topo.pillar_schedule(8, 512, 64, 128, 32)
    arr = _layers(plan)
    need = lib.topo_layers_workspace_bytes(ctypes.byref(p), arr, 8)
    # the largest of the layers' own needs (a dense layer or the widest decode layer)
    dense = lib.topo_workspace_bytes(ctypes.byref(_p(W=0, k=0)), 3)
    widest = lib.topo_workspace_bytes(ctypes.byref(_p(W=plan[1][1], k=plan[1][2])), 0)
    assert need == max(16, dense, widest) > 0
    ws = ctypes.c_void_p(1 << 40)
    assert lib.topo_attn_decode_layers(ctypes.byref(p), None, 8, ws, need, None) == -1
    assert lib.topo_attn_decode_layers(ctypes.byref(p), arr, 0, ws, need, None) == -1
    assert lib.topo_attn_decode_layers(ctypes.byref(p), arr, 8, ws, need - 1, None) == -3
    bad = _layers(plan)
    bad[5].W = -1
    assert lib.topo_layers_workspace_bytes(ctypes.byref(p), bad, 8) == 0
    assert lib.topo_attn_decode_layers(ctypes.byref(p), bad, 8, ws, need, None) == -1
    bad = _layers(plan)
    bad[3].reserved = 1
    assert lib.topo_attn_decode_layers(ctypes.byref(p), bad, 8, ws, need, None) == -1
    bad = _layers(plan)
    bad[2].v_cache = (1 << 40) + 8
    assert lib.topo_attn_decode_layers(ctypes.byref(p), bad, 8, ws, need, None) == -1
    assert lib.topo_attn_decode_layers(ctypes.byref(_p(n_q=2, q_pos0=0)), arr, 8, ws, need, None) == -1
