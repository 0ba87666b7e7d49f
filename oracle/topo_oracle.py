"""CPU oracle for Topological Attention over the condensate set (test infrastructure only).

Source: "The Condensate Theorem: Transformers are O(n), Not O(n^2)", the gist.science explainer
pages of arXiv 2602.06317 (zh, fr, hi, ar, ko). Citations below name a page by its language code
and the part of that page: "pop" is the popular explainer at the top of the page, "T§n" is
section n of the technical summary under it.

What the method computes, per query i (zh T§3 "研究方法"; fr T§2-§3; ko T§2-§3):
  * the condensate set C_i = anchor (position 0) ∪ the W most recent tokens ∪ the top-k
    positions by the score Q·K^T, recomputed for every query (ko T§3 "동적 선택");
  * attention restricted to C_i: a softmax over the positions in C_i only, then the
    softmax-weighted sum of their V rows (fr T§3).
The pages claim that the positions left out carry softmax weights below the float32 ulp, so the
set output equals dense attention bit for bit on trained models (zh T§2; hi T§2; ar T§2).

This is a plain, slow definition written out in float64. It is used by the tests, by the
smoke check and by the benchmark's CPU-baseline leg, and by nothing else: the GPU path never
calls it, and it shares no code with the GPU path.

Readings where the pages leave the arithmetic open (each is a choice, not something the pages fix):
  * Score: s_j = sum over t = 0..d-1 of q_t * k_{j,t}, each product and each partial sum in
    float64, summed in ascending t from +0.0. Products of float32 or bfloat16 values are exact
    in float64, so only the additions round.
  * Window: the W positions max(0, p-W+1) .. p, the query's own position included.
  * Top-k runs over the candidates, the visible keys outside the anchor and the window: [1, p-W]
    when causal. It ranks by the raw score s (the positive softmax scale does not change the real
    order), higher score first and, on equal scores, lower position first. If there are at most k
    candidates, all are taken.
  * Softmax in float64 on z_j = scale * s_j (scale widened from its float32 value), with
    w_j = exp(z_j - max z). Z = sum of w_j and N = sum of w_j * v_j, both summed in ascending j;
    the output is N / Z rounded once to float32.
  * GQA: query head h reads kv head floor(h / G), G = Hq / Hkv, and selects its own set.
  * GQA, shared selection (a variant; the pages name GQA without detail): one set per (batch,
    kv head) for all G query heads of the group. A key's group score is the largest score any of
    the group's heads gives it; the top-k ranks group scores as above; each head then takes the
    softmax of its own scores over the shared set.
  * Non-causal: every key 0..n-1 is visible; the window is still the W positions ending at p.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "canonical_scores", "condensate_set", "softmax_weighted_v", "attend", "dense_attend",
    "omitted_mass", "certified_components", "ulp_distance_f32", "topo_attn_decode",
    "topo_attn_rows", "dense_decode", "certificate_bound", "CERT_RHO", "KEY_BLOCK",
    "group_scores", "topo_attn_decode_group",
]

# A query is certified when its bound on the omitted softmax mass is below the float32 rounding
# unit: the set then carries the dense softmax to float32 precision (the exactness claim of zh T§2
# and hi T§2, excluded weights below float32 precision).
CERT_RHO = 2.0 ** -24

# Keys are processed in slices of this many rows only to bound memory; every key's score is an
# independent sum, so the slice size does not change any result.
KEY_BLOCK = 16384


def canonical_scores(q: np.ndarray, K: np.ndarray) -> np.ndarray:
    """Scores of one or several queries against every key.

    q: (d,) or (G, d); K: (n, d). Values must be float32-representable (float32 or bfloat16 data).
    Returns float64 (n,) or (G, n): s_j = sum_t q_t * k_{j,t}, float64, ascending t from +0.0.
    The score is the Q·K^T of zh T§3 (dynamic long-range selection) and ko T§3.
    """
    q64 = np.atleast_2d(np.asarray(q, dtype=np.float64))
    K = np.asarray(K)
    n, d = K.shape
    if q64.shape[1] != d:
        raise ValueError("q and K disagree on d")
    out = np.empty((q64.shape[0], n), dtype=np.float64)
    for j0 in range(0, n, KEY_BLOCK):
        Kt = np.array(K[j0:j0 + KEY_BLOCK].T, dtype=np.float64, order="C")   # (d, m)
        for h in range(q64.shape[0]):
            acc = np.zeros(Kt.shape[1], dtype=np.float64)
            for t in range(d):
                acc += q64[h, t] * Kt[t]
            out[h, j0:j0 + Kt.shape[1]] = acc
    return out[0] if np.ndim(q) == 1 else out


def condensate_set(s: np.ndarray, p: int, W: int, k: int, causal: bool = True):
    """The condensate set of a query at position p, given the scores s of all n keys.

    zh T§3 lists its three parts: the anchor (position 0, the attention sink), the local window of
    the most recent W tokens, and the k positions with the highest Q·K^T scores; fr T§2 names the
    same three. Returns (C, T): C is every position of the set, ascending (int64); T is the top-k
    part in rank order.
    """
    n = s.shape[0]
    if not 0 <= p < n:
        raise ValueError("query position outside the key range")
    vis_hi = p if causal else n - 1
    w_lo = max(0, p - W + 1)
    pos = np.arange(vis_hi + 1)
    in_window = (pos >= w_lo) & (pos <= p)
    cand = pos[(pos != 0) & ~in_window]
    # Higher score first; the stable sort keeps ascending position among equal scores.
    order = np.argsort(-s[cand], kind="stable")
    T = cand[order[:min(k, cand.size)]]
    members = np.zeros(vis_hi + 1, dtype=bool)
    members[0] = True
    members[w_lo:p + 1] = True
    members[T] = True
    return np.flatnonzero(members).astype(np.int64), T.astype(np.int64)


def softmax_weighted_v(s_sel: np.ndarray, V_sel: np.ndarray, scale: float):
    """Softmax over the given positions and the weighted sum of their V rows (fr T§3).

    s_sel: (m,) float64 scores in ascending position order; V_sel: (m, d) values.
    Returns (o float64 (d,), Z, zmax): o = sum_j w_j v_j / sum_j w_j with w_j = exp(z_j - zmax),
    z_j = scale * s_j; sums run sequentially in ascending position.
    """
    z = np.float64(scale) * np.asarray(s_sel, dtype=np.float64)
    zmax = z.max()
    w = np.exp(z - zmax)
    Z = np.cumsum(w)[-1]
    N = np.cumsum(w[:, None] * np.asarray(V_sel, dtype=np.float64), axis=0)[-1]
    return N / Z, Z, zmax


def attend(q, K, V, p: int, W: int, k: int, scale: float, causal: bool = True, s=None):
    """Topological attention of one query (zh T§3, fr T§3).

    q: (d,), K, V: (n, d). Returns (o float32 (d,), C, s) with s the scores of every key.
    """
    if s is None:
        s = canonical_scores(q, K)
    C, _ = condensate_set(s, p, W, k, causal)
    o, _, _ = softmax_weighted_v(s[C], np.asarray(V)[C], scale)
    return o.astype(np.float32), C, s


def dense_attend(q, K, V, p: int, scale: float, causal: bool = True, s=None):
    """Plain softmax attention of one query over every visible key, float64 (the comparator the
    exactness claim is stated against, zh T§2; also one pillar layer, zh T§3)."""
    if s is None:
        s = canonical_scores(q, K)
    vis_hi = p if causal else s.shape[0] - 1
    Vv = np.asarray(V)[:vis_hi + 1]
    z = np.float64(scale) * s[:vis_hi + 1]
    zmax = z.max()
    w = np.exp(z - zmax)
    Z = np.cumsum(w)[-1]
    N = np.zeros(Vv.shape[1], dtype=np.float64)
    for j0 in range(0, vis_hi + 1, KEY_BLOCK):
        blk = w[j0:j0 + KEY_BLOCK, None] * np.asarray(Vv[j0:j0 + KEY_BLOCK], dtype=np.float64)
        N = np.cumsum(np.vstack([N[None, :], blk]), axis=0)[-1]
    return N / Z


def omitted_mass(s: np.ndarray, C: np.ndarray, p: int, scale: float, causal: bool = True) -> float:
    """rho = softmax mass of the visible positions outside C, relative to the dense total.

    The exactness claim (zh T§2; hi T§2, excluded weights typically below 1e-7) is that rho is
    below the float32 rounding unit on trained models.
    """
    vis_hi = p if causal else s.shape[0] - 1
    z = np.float64(scale) * s[:vis_hi + 1]
    w = np.exp(z - z.max())
    inside = np.zeros(vis_hi + 1, dtype=bool)
    inside[C] = True
    return float(w[~inside].sum() / w.sum())


def certificate_bound(s: np.ndarray, p: int, W: int, k: int, scale: float, causal: bool = True) -> float:
    """An upper bound on omitted_mass from what is known once the set is chosen.

    Every candidate left out of the set scores at most s_k, the lowest score of the top-k part,
    so the omitted mass relative to the dense total is at most
        rho_hat = (number of omitted candidates) * exp(scale * s_k - zmax) / Z_C,
    with zmax and Z_C the softmax maximum and sum over the set (as in softmax_weighted_v). It is 0
    when no candidate is left out, and +inf when candidates are left out with k = 0 (no top-k part
    to bound them). Reading: the pages state the claim (zh T§2, hi T§2) but give no test; this is
    the plainest bound the selected scores support.
    """
    C, T = condensate_set(s, p, W, k, causal)
    vis_hi = p if causal else s.shape[0] - 1
    w_lo = max(0, p - W + 1)
    pos = np.arange(vis_hi + 1)
    n_cand = int(((pos != 0) & ~((pos >= w_lo) & (pos <= p))).sum())
    n_omit = n_cand - T.size
    if n_omit <= 0:
        return 0.0
    if T.size == 0:
        return float("inf")
    z = np.float64(scale) * np.asarray(s[C], dtype=np.float64)
    zmax = z.max()
    Z = np.cumsum(np.exp(z - zmax))[-1]
    s_k = float(np.min(s[T]))
    return float(n_omit * np.exp(np.float64(scale) * s_k - zmax) / Z)


def certified_components(o_set: np.ndarray, rho: float, vmax_out: np.ndarray) -> np.ndarray:
    """Components where dropping the omitted positions provably moves the exact output by less
    than a quarter of its float32 spacing.

    With rho the omitted mass ratio, |o_dense - o_set| <= rho * (|o_set| + max_{j not in C} |v_j|)
    per component. A move below a quarter spacing keeps the two float32 roundings at most one ulp
    apart, also across a binade edge.
    """
    o = np.abs(np.asarray(o_set, dtype=np.float64))
    bound = rho * (o + np.asarray(vmax_out, dtype=np.float64))
    spacing = np.spacing(o.astype(np.float32)).astype(np.float64)
    return bound < 0.25 * spacing


def ulp_distance_f32(a, b) -> np.ndarray:
    """Number of float32 values between a and b (0 = identical bits, ±0 equal)."""
    def ordered(x):
        i = np.asarray(x, dtype=np.float32).view(np.int32).astype(np.int64)
        return np.where(i < 0, -(i & 0x7FFFFFFF), i)
    return np.abs(ordered(a) - ordered(b))


def _kv_head(h: int, Hq: int, Hkv: int) -> int:
    return h // (Hq // Hkv)


def topo_attn_decode(q, K, V, W: int, k: int, scale: float, causal: bool = True, q_pos=None,
                     heads=None):
    """Topological attention of one query per (batch, query head).

    q: (B, Hq, d) or (B, Hq, 1, d); K, V: (B, Hkv, n, d); float32 values.
    q_pos: position of the query (default n-1, the newest token of the cache).
    heads: optional list of (b, h) to compute; the others are left as NaN / -1.
    Returns (out float32 (B, Hq, d), sel_idx int32 (B, Hq, 1+W+k) ascending and -1 padded,
    sel_count int32 (B, Hq)).
    """
    q = np.asarray(q)
    if q.ndim == 4:
        q = q[:, :, 0, :]
    B, Hq, d = q.shape
    _, Hkv, n, _ = K.shape
    p = n - 1 if q_pos is None else int(q_pos)
    out = np.full((B, Hq, d), np.nan, dtype=np.float32)
    sel = np.full((B, Hq, 1 + W + k), -1, dtype=np.int32)
    cnt = np.full((B, Hq), -1, dtype=np.int32)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        g = _kv_head(h, Hq, Hkv)
        o, C, _ = attend(q[b, h], K[b, g], V[b, g], p, W, k, scale, causal)
        out[b, h] = o
        sel[b, h, :C.size] = C
        cnt[b, h] = C.size
    return out, sel, cnt


def group_scores(s_heads: np.ndarray) -> np.ndarray:
    """Group score of every key for a shared selection: the largest of the group's per-head
    scores (s_heads: (G, n) float64)."""
    return np.max(np.asarray(s_heads, dtype=np.float64), axis=0)


def topo_attn_decode_group(q, K, V, W: int, k: int, scale: float, causal: bool = True, q_pos=None,
                           groups=None):
    """Topological attention with one condensate set per (batch, kv head), shared by the group's
    query heads: the set of the group scores (largest per-head score of each key), then each
    head's softmax of its own scores over it (the GQA shared-selection reading above).

    q: (B, Hq, d) or (B, Hq, 1, d); K, V: (B, Hkv, n, d). groups: optional list of (b, g).
    Returns (out float32 (B, Hq, d), sel_idx int32 (B, Hq, 1+W+k), sel_count int32 (B, Hq)); the
    heads of a group share sel_idx and sel_count.
    """
    q = np.asarray(q)
    if q.ndim == 4:
        q = q[:, :, 0, :]
    B, Hq, d = q.shape
    _, Hkv, n, _ = K.shape
    G = Hq // Hkv
    p = n - 1 if q_pos is None else int(q_pos)
    out = np.full((B, Hq, d), np.nan, dtype=np.float32)
    sel = np.full((B, Hq, 1 + W + k), -1, dtype=np.int32)
    cnt = np.full((B, Hq), -1, dtype=np.int32)
    todo = groups if groups is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in todo:
        heads = range(g * G, (g + 1) * G)
        s_heads = np.stack([canonical_scores(q[b, h], K[b, g]) for h in heads])
        C, _ = condensate_set(group_scores(s_heads), p, W, k, causal)
        for i, h in enumerate(heads):
            o, _, _ = softmax_weighted_v(s_heads[i][C], np.asarray(V[b, g])[C], scale)
            out[b, h] = o.astype(np.float32)
            sel[b, h, :C.size] = C
            cnt[b, h] = C.size
    return out, sel, cnt


def topo_attn_rows(Q, K, V, rows, W: int, k: int, scale: float, causal: bool = True, q_pos0: int = 0):
    """Topological attention for selected query rows of a many-query (prefill) call.

    Q: (Hq, n_q, d); K, V: (Hkv, n, d) for one batch entry. rows: iterable of (h, i) with query i
    at position q_pos0 + i. Returns {(h, i): (o float32 (d,), C)}.
    """
    Hq = Q.shape[0]
    Hkv = K.shape[0]
    res = {}
    for h, i in rows:
        g = _kv_head(h, Hq, Hkv)
        p = q_pos0 + i
        o, C, _ = attend(Q[h, i], K[g], V[g], p, W, k, scale, causal)
        res[(h, i)] = (o, C)
    return res


def dense_decode(q, K, V, scale: float, causal: bool = True, q_pos=None, heads=None):
    """Dense attention of one query per (batch, query head): the pillar layer of zh T§3."""
    q = np.asarray(q)
    if q.ndim == 4:
        q = q[:, :, 0, :]
    B, Hq, d = q.shape
    _, Hkv, n, _ = K.shape
    p = n - 1 if q_pos is None else int(q_pos)
    out = np.full((B, Hq, d), np.nan, dtype=np.float32)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        g = _kv_head(h, Hq, Hkv)
        out[b, h] = dense_attend(q[b, h], K[b, g], V[b, g], p, scale, causal).astype(np.float32)
    return out
