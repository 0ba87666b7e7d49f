"""Topological Attention over the condensate set on AMD MI355X (gfx950).

Python binding of libtopo_attn.so, the C ABI declared in include/topo_attn.h. Argument marshalling
only: every step of the computation runs in the library's HIP kernels. PyTorch supplies device
memory and the current stream. There is no fallback: if the library is missing or a call fails,
the call raises.

Method: "The Condensate Theorem: Transformers are O(n), Not O(n^2)" (gist.science explainers of
arXiv 2602.06317). Per query, attention runs over the anchor (position 0), the W most recent
tokens and the k keys with the highest Q.K^T scores (zh page, technical summary §3; fr page,
technical summary §3).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "TopoError", "load_library", "library_path", "topo_workspace_bytes", "topo_attn_decode",
    "topo_attn_prefill", "topo_select", "topo_attn_dense", "topo_bw_probe", "topo_strerror",
    "topo_attn_decode_timed", "topo_attn_prefill_timed", "topo_attn_decode_certified",
    "topo_attn_decode_ragged", "topo_kv_append", "topo_attn_decode_layers", "pillar_schedule",
    "topo_check_finite", "topo_workspace_view", "WorkspaceView", "topo_attn_decode_noalloc",
    "TOPO_NOALLOC_MAX_BYTES",
    "TOPO_FLAG_EXACT_SELECT", "TOPO_FLAG_DENSE_FALLBACK", "TOPO_FLAG_GROUP_SELECT", "TOPO_CERT_RHO", "TOPO_MAX_SET", "EXPORTS",
    "TOPO_PATH_NONE", "TOPO_PATH_ALL", "TOPO_PATH_FAST", "TOPO_PATH_BAND", "TOPO_PATH_EXACT_ASKED",
    "TOPO_PATH_EXACT_OVERFLOW", "TOPO_PATH_EXACT_CROWDED", "PATH_NAMES",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libtopo_attn.so")

TOPO_F32, TOPO_BF16 = 0, 1
TOPO_OP_DECODE, TOPO_OP_PREFILL, TOPO_OP_SELECT, TOPO_OP_DENSE, TOPO_OP_DECODE_CERTIFIED = 0, 1, 2, 3, 4
TOPO_OP_DECODE_RAGGED = 5
TOPO_FLAG_EXACT_SELECT = 1
TOPO_FLAG_DENSE_FALLBACK = 2
TOPO_FLAG_GROUP_SELECT = 4
TOPO_CERT_RHO = 2.0 ** -24
TOPO_MAX_SET = 4096
TOPO_NOALLOC_MAX_BYTES = 32 << 20
TOPO_PATH_NONE, TOPO_PATH_ALL, TOPO_PATH_FAST, TOPO_PATH_BAND = 0, 1, 2, 3
TOPO_PATH_EXACT_ASKED, TOPO_PATH_EXACT_OVERFLOW, TOPO_PATH_EXACT_CROWDED = 4, 5, 6
PATH_NAMES = {0: "none", 1: "all", 2: "fast", 3: "band", 4: "exact_asked", 5: "exact_overflow", 6: "exact_crowded"}
EXPORTS = ("topo_workspace_bytes", "topo_attn_decode", "topo_attn_decode_noalloc", "topo_attn_decode_timed",
           "topo_attn_decode_certified",
           "topo_attn_decode_ragged", "topo_kv_append", "topo_attn_decode_layers", "topo_layers_workspace_bytes",
           "topo_pillar_plan", "topo_attn_prefill", "topo_attn_prefill_timed", "topo_select", "topo_attn_dense",
           "topo_check_finite", "topo_workspace_view", "topo_bw_probe", "topo_strerror")


class TopoLayer(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("sel_idx", ctypes.c_void_p), ("sel_count", ctypes.c_void_p),
                ("W", ctypes.c_int32), ("k", ctypes.c_int32), ("pillar", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class WorkspaceView(ctypes.Structure):
    """topo_ws_view_t: where a call leaves its candidate lists and selection paths in the workspace."""
    _fields_ = [("queries", ctypes.c_int64), ("lists", ctypes.c_int64), ("slots", ctypes.c_int64),
                ("count_offset", ctypes.c_size_t), ("entry_offset", ctypes.c_size_t),
                ("eps_offset", ctypes.c_size_t), ("path_offset", ctypes.c_size_t),
                ("path_stride", ctypes.c_size_t), ("eps_coef", ctypes.c_float), ("count_split", ctypes.c_int32)]


class TopoError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {topo_strerror(status)} (status {status})")
        self.status = status


class TopoParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("n_ctx", ctypes.c_int64), ("n_q", ctypes.c_int64),
                ("q_pos0", ctypes.c_int64), ("W", ctypes.c_int32), ("k", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libtopo_attn.so (built in-tree by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    # torch first: it ships its own HIP runtime, whose soname the library's dependency matches, so
    # both then share one runtime (and one HSA runtime). Loaded the other way round, the process
    # would hold two runtimes, and torch's streams and allocations passed to the library would
    # belong to the other one.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(p)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    P = ctypes.POINTER(TopoParams)
    lib.topo_workspace_bytes.argtypes = [P, i32]
    lib.topo_workspace_bytes.restype = sz
    for name in ("topo_attn_decode", "topo_attn_prefill"):
        f = getattr(lib, name)
        f.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        f.restype = i32
    lib.topo_attn_decode_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    lib.topo_attn_decode_noalloc.restype = i32
    lib.topo_attn_decode_timed.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.topo_attn_decode_timed.restype = i32
    lib.topo_attn_prefill_timed.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.topo_attn_prefill_timed.restype = i32
    lib.topo_attn_decode_certified.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.topo_attn_decode_certified.restype = i32
    lib.topo_attn_decode_ragged.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.topo_attn_decode_ragged.restype = i32
    lib.topo_kv_append.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.topo_kv_append.restype = i32
    LP = ctypes.POINTER(TopoLayer)
    lib.topo_layers_workspace_bytes.argtypes = [P, LP, i32]
    lib.topo_layers_workspace_bytes.restype = sz
    lib.topo_attn_decode_layers.argtypes = [P, LP, i32, vp, sz, vp]
    lib.topo_attn_decode_layers.restype = i32
    lib.topo_select.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
    lib.topo_select.restype = i32
    lib.topo_attn_dense.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
    lib.topo_attn_dense.restype = i32
    lib.topo_pillar_plan.argtypes = [i32, i32, i32, i32, i32, LP]
    lib.topo_pillar_plan.restype = i32
    lib.topo_check_finite.argtypes = [vp, sz, i32, vp, vp]
    lib.topo_check_finite.restype = i32
    lib.topo_workspace_view.argtypes = [P, i32, ctypes.POINTER(WorkspaceView)]
    lib.topo_workspace_view.restype = i32
    lib.topo_bw_probe.argtypes = [vp, sz, vp, vp]
    lib.topo_bw_probe.restype = i32
    lib.topo_strerror.argtypes = [i32]
    lib.topo_strerror.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def topo_strerror(status: int) -> str:
    return load_library().topo_strerror(int(status)).decode()


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return TOPO_F32
    if t.dtype == torch.bfloat16:
        return TOPO_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _params(q, k, W, topk, softmax_scale, causal, q_pos0, flags) -> TopoParams:
    B, Hq, n_q, d = q.shape
    Bk, Hkv, n_ctx, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree")
    return TopoParams(B, Hq, Hkv, d, n_ctx, n_q, int(q_pos0), int(W), int(topk), int(bool(causal)),
                      float(softmax_scale), _dtype_code(q), int(flags))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check_tensors(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def topo_workspace_bytes(q, k, W: int, topk: int, softmax_scale: float, causal: bool = True,
                         q_pos0: int | None = None, op: int = TOPO_OP_DECODE, flags: int = 0) -> int:
    q4 = q if q.dim() == 4 else q.unsqueeze(2)
    if q_pos0 is None:
        q_pos0 = k.shape[2] - q4.shape[2]
    p = _params(q4, k, W, topk, softmax_scale, causal, q_pos0, flags)
    return int(load_library().topo_workspace_bytes(ctypes.byref(p), op))


def _workspace(nbytes, device, workspace):
    torch = _torch()
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise TopoError(-3, "workspace")
        return workspace
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def _attn(name, q, k, v, W, topk, softmax_scale, causal, q_pos0, flags, out, sel_idx, sel_count,
          workspace, stream, want_sets):
    torch = _torch()
    lib = load_library()
    q4 = q if q.dim() == 4 else q.unsqueeze(2)
    if q_pos0 is None:
        q_pos0 = k.shape[2] - q4.shape[2]
    p = _params(q4, k, W, topk, softmax_scale, causal, q_pos0, flags)
    _check_tensors(q4, k, v)
    B, Hq, n_q, d = q4.shape
    S = 1 + int(W) + int(topk)
    op = TOPO_OP_DECODE if name == "topo_attn_decode" else TOPO_OP_PREFILL
    nbytes = lib.topo_workspace_bytes(ctypes.byref(p), op)
    if nbytes == 0:
        raise TopoError(-1, f"{name}: parameters rejected")
    ws = _workspace(nbytes, q4.device, workspace)
    if out is None:
        out = torch.empty((B, Hq, n_q, d), dtype=torch.float32, device=q4.device)
    if want_sets:
        if sel_idx is None:
            sel_idx = torch.empty((B, Hq, n_q, S), dtype=torch.int32, device=q4.device)
        if sel_count is None:
            sel_count = torch.empty((B, Hq, n_q), dtype=torch.int32, device=q4.device)
    _check_tensors(out, sel_idx, sel_count)
    rc = getattr(lib, name)(ctypes.byref(p), _ptr(q4), _ptr(k), _ptr(v), _ptr(out), _ptr(sel_idx),
                            _ptr(sel_count), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(stream))
    if rc != 0:
        raise TopoError(rc, name)
    return out, sel_idx, sel_count


def topo_attn_decode(q, k, v, W: int, topk: int, softmax_scale: float, causal: bool = True,
                     q_pos0: int | None = None, flags: int = 0, out=None, sel_idx=None, sel_count=None,
                     workspace=None, stream=None, want_sets: bool = True):
    """One query per (batch, query head). q: (B, Hq, d) or (B, Hq, 1, d); k, v: (B, Hkv, n, d).
    q_pos0 defaults to n-1 (the newest token). Returns (out f32 (B,Hq,1,d), sel_idx, sel_count)."""
    return _attn("topo_attn_decode", q, k, v, W, topk, softmax_scale, causal, q_pos0, flags, out, sel_idx,
                 sel_count, workspace, stream, want_sets)


def topo_attn_decode_noalloc(q, k, v, W: int, topk: int, softmax_scale: float, causal: bool = True,
                             q_pos0: int | None = None, flags: int = 0, out=None, sel_idx=None, sel_count=None,
                             stream=None):
    """topo_attn_decode with no workspace argument: the library uses its own static per-GPU buffer
    (topo_attn_decode_noalloc; calls that overlap on one GPU race). Output and set tensors are
    created here when not given; pass them to allocate nothing at all."""
    torch = _torch()
    lib = load_library()
    q4 = q if q.dim() == 4 else q.unsqueeze(2)
    if q_pos0 is None:
        q_pos0 = k.shape[2] - q4.shape[2]
    p = _params(q4, k, W, topk, softmax_scale, causal, q_pos0, flags)
    _check_tensors(q4, k, v)
    B, Hq, n_q, d = q4.shape
    if out is None:
        out = torch.empty((B, Hq, n_q, d), dtype=torch.float32, device=q4.device)
    if sel_idx is None:
        sel_idx = torch.empty((B, Hq, n_q, 1 + int(W) + int(topk)), dtype=torch.int32, device=q4.device)
    if sel_count is None:
        sel_count = torch.empty((B, Hq, n_q), dtype=torch.int32, device=q4.device)
    _check_tensors(out, sel_idx, sel_count)
    rc = lib.topo_attn_decode_noalloc(ctypes.byref(p), _ptr(q4), _ptr(k), _ptr(v), _ptr(out), _ptr(sel_idx),
                                      _ptr(sel_count), _stream(stream))
    if rc != 0:
        raise TopoError(rc, "topo_attn_decode_noalloc")
    return out, sel_idx, sel_count


def _attn_timed(name, op, q, k, v, W, topk, softmax_scale, scan_begin, scan_end, causal, q_pos0, flags, out,
                sel_idx, sel_count, workspace, stream):
    torch = _torch()
    lib = load_library()
    q4 = q if q.dim() == 4 else q.unsqueeze(2)
    if q_pos0 is None:
        q_pos0 = k.shape[2] - q4.shape[2]
    p = _params(q4, k, W, topk, softmax_scale, causal, q_pos0, flags)
    _check_tensors(q4, k, v)
    B, Hq, n_q, d = q4.shape
    nbytes = lib.topo_workspace_bytes(ctypes.byref(p), op)
    if nbytes == 0:
        raise TopoError(-1, f"{name}: parameters rejected")
    ws = _workspace(nbytes, q4.device, workspace)
    if out is None:
        out = torch.empty((B, Hq, n_q, d), dtype=torch.float32, device=q4.device)
    rc = getattr(lib, name)(ctypes.byref(p), _ptr(q4), _ptr(k), _ptr(v), _ptr(out), _ptr(sel_idx),
                            _ptr(sel_count), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(stream),
                            ctypes.c_void_p(scan_begin.cuda_event), ctypes.c_void_p(scan_end.cuda_event))
    if rc != 0:
        raise TopoError(rc, name)
    return out, sel_idx, sel_count


def topo_attn_decode_timed(q, k, v, W: int, topk: int, softmax_scale: float, scan_begin, scan_end,
                           causal: bool = True, q_pos0: int | None = None, flags: int = 0, out=None,
                           sel_idx=None, sel_count=None, workspace=None, stream=None):
    """topo_attn_decode that also records the torch.cuda.Event pair scan_begin / scan_end around the
    key-scan kernel on the call's stream (both events must have been recorded once, so that their
    HIP handles exist). Read the scan time with scan_begin.elapsed_time(scan_end)."""
    return _attn_timed("topo_attn_decode_timed", TOPO_OP_DECODE, q, k, v, W, topk, softmax_scale, scan_begin,
                       scan_end, causal, q_pos0, flags, out, sel_idx, sel_count, workspace, stream)


def topo_attn_prefill_timed(q, k, v, W: int, topk: int, softmax_scale: float, scan_begin, scan_end,
                            causal: bool = True, q_pos0: int | None = None, flags: int = 0, out=None,
                            sel_idx=None, sel_count=None, workspace=None, stream=None):
    """topo_attn_prefill that also records scan_begin / scan_end around the matrix-core key scan."""
    return _attn_timed("topo_attn_prefill_timed", TOPO_OP_PREFILL, q, k, v, W, topk, softmax_scale, scan_begin,
                       scan_end, causal, q_pos0, flags, out, sel_idx, sel_count, workspace, stream)


def _check_pos(pos, B):
    torch = _torch()
    if pos.dtype != torch.int64 or pos.dim() != 1 or pos.shape[0] != B:
        raise ValueError(f"pos must be an int64 device tensor of shape ({B},)")
    _check_tensors(pos)


def topo_attn_decode_ragged(q, k, v, pos, W: int, topk: int, softmax_scale: float, flags: int = 0, out=None,
                            sel_idx=None, sel_count=None, workspace=None, stream=None):
    """Decode of sequences of different lengths: the query of batch element b sits at position
    pos[b] (int64 device tensor (B,)) of its own cache and sees keys 0..pos[b]. q: (B, Hq, d) or
    (B, Hq, 1, d); k, v: (B, Hkv, n_ctx, d). Returns (out f32 (B,Hq,1,d), sel_idx, sel_count)."""
    torch = _torch()
    lib = load_library()
    q4 = q if q.dim() == 4 else q.unsqueeze(2)
    p = _params(q4, k, W, topk, softmax_scale, True, k.shape[2] - 1, flags)
    _check_tensors(q4, k, v)
    B, Hq, n_q, d = q4.shape
    _check_pos(pos, B)
    nbytes = lib.topo_workspace_bytes(ctypes.byref(p), TOPO_OP_DECODE_RAGGED)
    if nbytes == 0:
        raise TopoError(-1, "topo_attn_decode_ragged: parameters rejected")
    ws = _workspace(nbytes, q4.device, workspace)
    if out is None:
        out = torch.empty((B, Hq, n_q, d), dtype=torch.float32, device=q4.device)
    if sel_idx is None:
        sel_idx = torch.empty((B, Hq, n_q, 1 + int(W) + int(topk)), dtype=torch.int32, device=q4.device)
    if sel_count is None:
        sel_count = torch.empty((B, Hq, n_q), dtype=torch.int32, device=q4.device)
    _check_tensors(out, sel_idx, sel_count)
    rc = lib.topo_attn_decode_ragged(ctypes.byref(p), _ptr(pos), _ptr(q4), _ptr(k), _ptr(v), _ptr(out),
                                     _ptr(sel_idx), _ptr(sel_count), _ptr(ws), ctypes.c_size_t(ws.numel()),
                                     _stream(stream))
    if rc != 0:
        raise TopoError(rc, "topo_attn_decode_ragged")
    return out, sel_idx, sel_count


def topo_kv_append(k_cache, v_cache, k_new, v_new, pos, stream=None):
    """Write one token's key and value rows per (batch, kv head) into the caches at row pos[b].
    k_cache, v_cache: (B, Hkv, n_ctx, d); k_new, v_new: (B, Hkv, d) (or (B, Hkv, 1, d)), same
    dtype; pos: int64 device tensor (B,)."""
    lib = load_library()
    B, Hkv, n_ctx, d = k_cache.shape
    k3 = k_new.reshape(B, Hkv, d)
    v3 = v_new.reshape(B, Hkv, d)
    if v_cache.shape != k_cache.shape or k3.dtype != k_cache.dtype or v3.dtype != k_cache.dtype:
        raise ValueError("caches and new rows disagree in shape or dtype")
    _check_tensors(k_cache, v_cache, k3, v3)
    _check_pos(pos, B)
    p = TopoParams(B, Hkv, Hkv, d, n_ctx, 1, n_ctx - 1, 0, 0, 1, 1.0, _dtype_code(k_cache), 0)
    rc = lib.topo_kv_append(ctypes.byref(p), _ptr(pos), _ptr(k3), _ptr(v3), _ptr(k_cache), _ptr(v_cache),
                            _stream(stream))
    if rc != 0:
        raise TopoError(rc, "topo_kv_append")


def pillar_schedule(n_layers: int, W_first: int, k_first: int, W_last: int | None = None, k_last: int | None = None):
    """Per-layer plan of a decode step through n_layers attention layers, from the library's
    topo_pillar_plan: a list of (pillar, W, k). About one layer in sixteen is a pillar (dense)
    layer: max(1, round(L / 16)) of them, evenly spaced from layer 0. Every layer takes (W, k)
    interpolated linearly from (W_first, k_first) at layer 0 to (W_last, k_last) at the last
    layer, rounded: wider windows early, leaner sets late (zh page, technical summary §3)."""
    W_last = W_first if W_last is None else W_last
    k_last = k_first if k_last is None else k_last
    if n_layers < 1:
        raise ValueError("n_layers >= 1")
    arr = (TopoLayer * n_layers)()
    rc = load_library().topo_pillar_plan(int(n_layers), int(W_first), int(k_first), int(W_last), int(k_last), arr)
    if rc != 0:
        raise TopoError(rc, "topo_pillar_plan")
    return [(bool(arr[i].pillar), int(arr[i].W), int(arr[i].k)) for i in range(n_layers)]


def topo_check_finite(buf, flag=None, stream=None):
    """Set flag[0] (an int32 device tensor, not cleared here) to 1 if the float32 or bfloat16
    device tensor `buf` holds a NaN or an infinity. Returns flag (read it after synchronising)."""
    torch = _torch()
    if flag is None:
        flag = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check_tensors(buf, flag)
    rc = load_library().topo_check_finite(_ptr(buf), ctypes.c_size_t(buf.numel()), _dtype_code(buf), _ptr(flag),
                                          _stream(stream))
    if rc != 0:
        raise TopoError(rc, "topo_check_finite")
    return flag


def topo_workspace_view(q, k, W: int, topk: int, softmax_scale: float = 1.0, causal: bool = True,
                        q_pos0: int | None = None, op: int = TOPO_OP_DECODE, flags: int = 0) -> WorkspaceView:
    """Where a call with these arguments leaves the key scan's candidate lists and each query's
    selection path (TOPO_PATH_*) in its workspace (topo_workspace_view)."""
    q4 = q if q.dim() == 4 else q.unsqueeze(2)
    if q_pos0 is None:
        q_pos0 = k.shape[2] - q4.shape[2]
    p = _params(q4, k, W, topk, softmax_scale, causal, q_pos0, flags)
    v = WorkspaceView()
    rc = load_library().topo_workspace_view(ctypes.byref(p), int(op), ctypes.byref(v))
    if rc != 0:
        raise TopoError(rc, "topo_workspace_view")
    return v


def topo_attn_decode_layers(layers, plan, softmax_scale: float, q_pos0: int | None = None, flags: int = 0,
                            want_sets: bool = True, workspace=None, stream=None):
    """A decode step through a stack of attention layers, launched by one library call.
    layers: sequence of (q, k, v) per layer, q (B, Hq, d) or (B, Hq, 1, d), k and v (B, Hkv, n, d),
    all layers of one shape and dtype. plan: per layer (pillar, W, k), e.g. from pillar_schedule.
    Returns a list of (out f32 (B,Hq,1,d), sel_idx or None, sel_count or None) per layer (no sets
    for pillar layers)."""
    torch = _torch()
    lib = load_library()
    if len(layers) != len(plan) or not layers:
        raise ValueError("one plan entry per layer")
    q0 = layers[0][0]
    q04 = q0 if q0.dim() == 4 else q0.unsqueeze(2)
    k0 = layers[0][1]
    if q_pos0 is None:
        q_pos0 = k0.shape[2] - 1
    p = _params(q04, k0, 0, 0, softmax_scale, True, q_pos0, flags)
    B, Hq, _, d = q04.shape
    arr = (TopoLayer * len(layers))()
    results, keep = [], []
    for i, ((q, k, v), (pillar, W, kk)) in enumerate(zip(layers, plan)):
        q4 = q if q.dim() == 4 else q.unsqueeze(2)
        if q4.shape != q04.shape or k.shape != k0.shape or v.shape != k0.shape or q4.dtype != q04.dtype:
            raise ValueError(f"layer {i}: shapes or dtype differ from layer 0")
        _check_tensors(q4, k, v)
        out = torch.empty((B, Hq, 1, d), dtype=torch.float32, device=q4.device)
        sel = cnt = None
        if want_sets and not pillar:
            sel = torch.empty((B, Hq, 1, 1 + int(W) + int(kk)), dtype=torch.int32, device=q4.device)
            cnt = torch.empty((B, Hq, 1), dtype=torch.int32, device=q4.device)
        arr[i] = TopoLayer(q4.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           sel.data_ptr() if sel is not None else None, cnt.data_ptr() if cnt is not None else None,
                           int(W), int(kk), int(bool(pillar)), 0)
        keep.append(q4)
        results.append((out, sel, cnt))
    nbytes = lib.topo_layers_workspace_bytes(ctypes.byref(p), arr, len(layers))
    if nbytes == 0:
        raise TopoError(-1, "topo_attn_decode_layers: parameters rejected")
    ws = _workspace(nbytes, q04.device, workspace)
    rc = lib.topo_attn_decode_layers(ctypes.byref(p), arr, len(layers), _ptr(ws), ctypes.c_size_t(ws.numel()),
                                     _stream(stream))
    if rc != 0:
        raise TopoError(rc, "topo_attn_decode_layers")
    return results


def topo_attn_decode_certified(q, k, v, W: int, topk: int, softmax_scale: float, dense_fallback: bool = False,
                               causal: bool = True, q_pos0: int | None = None, flags: int = 0, out=None,
                               sel_idx=None, sel_count=None, rho=None, workspace=None, stream=None):
    """topo_attn_decode plus the exactness certificate: rho (B, Hq) float32, an upper bound on the
    softmax mass left out of each query's set. With dense_fallback, queries with
    rho >= TOPO_CERT_RHO get dense attention in out. Returns (out, sel_idx, sel_count, rho)."""
    torch = _torch()
    lib = load_library()
    q4 = q if q.dim() == 4 else q.unsqueeze(2)
    if q_pos0 is None:
        q_pos0 = k.shape[2] - q4.shape[2]
    if dense_fallback:
        flags |= TOPO_FLAG_DENSE_FALLBACK
    p = _params(q4, k, W, topk, softmax_scale, causal, q_pos0, flags)
    _check_tensors(q4, k, v)
    B, Hq, n_q, d = q4.shape
    nbytes = lib.topo_workspace_bytes(ctypes.byref(p), TOPO_OP_DECODE_CERTIFIED)
    if nbytes == 0:
        raise TopoError(-1, "topo_attn_decode_certified: parameters rejected")
    ws = _workspace(nbytes, q4.device, workspace)
    if out is None:
        out = torch.empty((B, Hq, n_q, d), dtype=torch.float32, device=q4.device)
    if sel_idx is None:
        sel_idx = torch.empty((B, Hq, n_q, 1 + int(W) + int(topk)), dtype=torch.int32, device=q4.device)
    if sel_count is None:
        sel_count = torch.empty((B, Hq, n_q), dtype=torch.int32, device=q4.device)
    if rho is None:
        rho = torch.empty((B, Hq), dtype=torch.float32, device=q4.device)
    rc = lib.topo_attn_decode_certified(ctypes.byref(p), _ptr(q4), _ptr(k), _ptr(v), _ptr(out), _ptr(sel_idx),
                                        _ptr(sel_count), _ptr(rho), _ptr(ws), ctypes.c_size_t(ws.numel()),
                                        _stream(stream))
    if rc != 0:
        raise TopoError(rc, "topo_attn_decode_certified")
    return out, sel_idx, sel_count, rho


def topo_attn_prefill(q, k, v, W: int, topk: int, softmax_scale: float, causal: bool = True,
                      q_pos0: int | None = None, flags: int = 0, out=None, sel_idx=None, sel_count=None,
                      workspace=None, stream=None, want_sets: bool = True):
    """n_q queries per (batch, query head) at positions q_pos0 .. q_pos0+n_q-1 (default: the last
    n_q positions; a whole prompt is q_pos0 = 0, n_q = n). q: (B, Hq, n_q, d)."""
    return _attn("topo_attn_prefill", q, k, v, W, topk, softmax_scale, causal, q_pos0, flags, out, sel_idx,
                 sel_count, workspace, stream, want_sets)


def topo_select(q, k, W: int, topk: int, softmax_scale: float = 1.0, causal: bool = True,
                q_pos0: int | None = None, flags: int = 0, sel_idx=None, sel_count=None, workspace=None,
                stream=None):
    """Condensate sets only. Returns (sel_idx int32 (B,Hq,n_q,1+W+k), sel_count int32 (B,Hq,n_q))."""
    torch = _torch()
    lib = load_library()
    q4 = q if q.dim() == 4 else q.unsqueeze(2)
    if q_pos0 is None:
        q_pos0 = k.shape[2] - q4.shape[2]
    p = _params(q4, k, W, topk, softmax_scale, causal, q_pos0, flags)
    _check_tensors(q4, k)
    B, Hq, n_q, d = q4.shape
    nbytes = lib.topo_workspace_bytes(ctypes.byref(p), TOPO_OP_SELECT)
    if nbytes == 0:
        raise TopoError(-1, "topo_select: parameters rejected")
    ws = _workspace(nbytes, q4.device, workspace)
    if sel_idx is None:
        sel_idx = torch.empty((B, Hq, n_q, 1 + int(W) + int(topk)), dtype=torch.int32, device=q4.device)
    if sel_count is None:
        sel_count = torch.empty((B, Hq, n_q), dtype=torch.int32, device=q4.device)
    rc = lib.topo_select(ctypes.byref(p), _ptr(q4), _ptr(k), _ptr(sel_idx), _ptr(sel_count), _ptr(ws),
                         ctypes.c_size_t(ws.numel()), _stream(stream))
    if rc != 0:
        raise TopoError(rc, "topo_select")
    return sel_idx, sel_count


def topo_attn_dense(q, k, v, softmax_scale: float, causal: bool = True, q_pos0: int | None = None,
                    out=None, workspace=None, stream=None):
    """Dense attention over every visible key (the pillar layer). Returns out f32 (B,Hq,n_q,d)."""
    torch = _torch()
    lib = load_library()
    q4 = q if q.dim() == 4 else q.unsqueeze(2)
    if q_pos0 is None:
        q_pos0 = k.shape[2] - q4.shape[2]
    p = _params(q4, k, 0, 0, softmax_scale, causal, q_pos0, 0)
    _check_tensors(q4, k, v)
    B, Hq, n_q, d = q4.shape
    nbytes = lib.topo_workspace_bytes(ctypes.byref(p), TOPO_OP_DENSE)
    if nbytes == 0:
        raise TopoError(-1, "topo_attn_dense: parameters rejected")
    ws = _workspace(nbytes, q4.device, workspace)
    if out is None:
        out = torch.empty((B, Hq, n_q, d), dtype=torch.float32, device=q4.device)
    rc = lib.topo_attn_dense(ctypes.byref(p), _ptr(q4), _ptr(k), _ptr(v), _ptr(out), _ptr(ws),
                             ctypes.c_size_t(ws.numel()), _stream(stream))
    if rc != 0:
        raise TopoError(rc, "topo_attn_dense")
    return out


def topo_bw_probe(buf, sink=None, stream=None):
    """Stream every byte of the device tensor `buf` once (read-bandwidth reference)."""
    torch = _torch()
    lib = load_library()
    if sink is None:
        sink = torch.zeros(4, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    rc = lib.topo_bw_probe(_ptr(buf), ctypes.c_size_t(nbytes - nbytes % 16), _ptr(sink), _stream(stream))
    if rc != 0:
        raise TopoError(rc, "topo_bw_probe")
    return sink
