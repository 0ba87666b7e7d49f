"""Seeded synthetic inputs for condensate-set attention.

Source: "The Condensate Theorem: Transformers are O(n), Not O(n^2)" (explainer pages on
gist.science for arXiv 2602.06317). The condensate set of a query is the anchor (position 0),
a window of the most recent tokens and a dynamic top-k by Q.K^T (zh page, technical summary §3
"研究方法"; fr page, technical summary §2). The workloads below give those three parts something
to find: a heavy anchor key (the attention sink, fr page, technical summary §2, which puts its
share of attention at 30-70 %), planted high-score keys far from the query (the "needle" that the
dynamic top-k must retrieve, zh page, technical summary §5) and N(0,1) bulk everywhere else.

This module only draws random numbers and shapes them. It holds none of the method's arithmetic
(no scores, no selection, no softmax), so the CPU oracle and the GPU path can both take their
inputs from here without sharing any of the computation they are compared on.

Recipe (every number here is the same on any machine):
* One ``numpy.random.SeedSequence(seed)`` per workload, ``seed = 1000 * config + trial``.
  It spawns one child per (batch, kv-head) group, so any group can be generated alone and a group
  is identical whether the others were generated or not.
* Within a group the draws come in this order: Q rows of the G query heads, K rows, V rows,
  then the positions and noise of the planted keys. All normals are float32 ``standard_normal``.
* bf16 tensors are rounded from the float32 values by round-to-nearest-even on the bit pattern,
  and are handed out as ``uint16`` bit arrays. Q has the dtype of K and V.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

__all__ = [
    "CONFIGS", "WorkloadSpec", "Workload", "spec", "make_workload", "gen_group",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "to_f32",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any((u & 0x7F800000) == 0x7F800000):
        raise ValueError("non-finite input")
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f32(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (float32, or uint16 bf16 bits) -> float32 values (exact)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32)
    raise ValueError(dtype)


@dataclass(frozen=True)
class WorkloadSpec:
    cfg: int
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    n_ctx: int
    mode: str            # "decode" (one query at position n_ctx-1) or "prefill" (every position)
    dtype: str           # "f32" or "bf16"
    W: int
    k: int
    beta: float = 1.0    # logit temperature: softmax_scale = beta / sqrt(d)
    anchor_gain: float = 0.0   # k_0 := anchor_gain * (unit mean query direction); 0 = plain N(0,1)
    planted: str = "none"      # "tiny" | "per_head" | "per_group" | "per_row" | "none"
    n_planted: int = 0         # tiny/per_head/per_group: keys per head or group; per_row: keys per row
    causal: bool = True

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_q(self) -> int:
        return self.n_ctx if self.mode == "prefill" else 1

    @property
    def q_pos0(self) -> int:
        return 0 if self.mode == "prefill" else self.n_ctx - 1

    @property
    def softmax_scale(self) -> np.float32:
        return np.float32(self.beta / math.sqrt(self.d))

    @property
    def set_size(self) -> int:
        return 1 + self.W + self.k


# The five workloads. Shapes follow the models the pages validate on (GPT-2, Mistral; zh page,
# technical summary §4) and the context lengths of its speed results (131K and 1M tokens, zh page,
# technical summary §5). beta=16 for the two long GQA decodes is the logit temperature that keeps
# the softmax mass left outside the set below 2^-24, the float32 half-ulp (the exactness claim of
# the zh page, technical summary §2); the oracle tests check that it does.
CONFIGS: dict[int, WorkloadSpec] = {
    1: WorkloadSpec(1, "tiny-decode", B=1, Hq=1, Hkv=1, d=64, n_ctx=1024, mode="decode", dtype="f32",
                    W=32, k=64, planted="tiny", n_planted=4),
    2: WorkloadSpec(2, "gpt2-small-decode", B=1, Hq=12, Hkv=12, d=64, n_ctx=4096, mode="decode",
                    dtype="f32", W=64, k=32, anchor_gain=8.0, planted="per_head", n_planted=16),
    3: WorkloadSpec(3, "causal-prefill", B=1, Hq=8, Hkv=8, d=128, n_ctx=8192, mode="prefill",
                    dtype="bf16", W=128, k=64, anchor_gain=6.0, planted="per_row", n_planted=8),
    4: WorkloadSpec(4, "mistral7b-gqa-decode-128k", B=4, Hq=32, Hkv=8, d=128, n_ctx=131072,
                    mode="decode", dtype="bf16", W=256, k=64, beta=16.0, anchor_gain=8.0,
                    planted="per_group", n_planted=32),
    5: WorkloadSpec(5, "gqa-decode-1m", B=1, Hq=32, Hkv=8, d=128, n_ctx=1 << 20, mode="decode",
                    dtype="bf16", W=512, k=64, beta=16.0, anchor_gain=8.0, planted="per_group",
                    n_planted=32),
}


def spec(cfg: int, **overrides) -> WorkloadSpec:
    """The spec of a config, optionally with fields replaced (smaller n_ctx, other W/k, ...)."""
    s = replace(CONFIGS[cfg], **overrides)
    if s.Hq % s.Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return s


def _unit(x: np.ndarray) -> np.ndarray:
    x64 = np.asarray(x, dtype=np.float64)
    return (x64 / np.linalg.norm(x64)).astype(np.float32)


def _distinct(rng: np.random.Generator, lo: int, hi: int, m: int) -> np.ndarray:
    """m distinct integers drawn uniformly from [lo, hi], ascending."""
    span = hi - lo + 1
    if m > span:
        raise ValueError(f"cannot draw {m} distinct positions from [{lo}, {hi}]")
    if span <= 4 * m:
        return np.sort(rng.permutation(span)[:m] + lo)
    out = np.unique(rng.integers(lo, hi + 1, size=m))
    while out.size < m:
        out = np.unique(np.concatenate([out, rng.integers(lo, hi + 1, size=m - out.size)]))
    return out


def gen_group(s: WorkloadSpec, trial: int, b: int, g: int):
    """Generate one (batch b, kv-head g) group.

    Returns (q, k, v, planted): q is (G, n_q, d), k and v are (n_ctx, d), all float32 values that
    are exactly representable in the workload dtype; planted maps a query head (global index) to
    the positions planted for it (decode), or for "per_row" to a (rows, positions) pair.
    """
    seed = 1000 * s.cfg + trial
    child = np.random.SeedSequence(seed).spawn(s.B * s.Hkv)[b * s.Hkv + g]
    rng = np.random.default_rng(child)
    G, n, d, nq = s.G, s.n_ctx, s.d, s.n_q
    q = rng.standard_normal((G, nq, d), dtype=np.float32)
    k = rng.standard_normal((n, d), dtype=np.float32)
    v = rng.standard_normal((n, d), dtype=np.float32)
    planted: dict = {}
    heads = [g * G + i for i in range(G)]
    cand_hi = n - 1 - s.W          # decode: the keys outside the anchor and the window are [1, n-1-W]

    if s.anchor_gain:
        if s.mode == "prefill":
            u = _unit(q.reshape(-1, d).astype(np.float64).mean(axis=0))
        else:
            u = _unit(q[:, 0, :].astype(np.float64).sum(axis=0))
        k[0] = np.float32(s.anchor_gain) * u

    if s.planted == "tiny":
        # k_p = q * 3/|q|^2 + noise, read literally (the query of this one-head decode).
        pos = _distinct(rng, 1, cand_hi, s.n_planted)
        qq = q[0, 0].astype(np.float64)
        base = (qq * (3.0 / float(qq @ qq))).astype(np.float32)
        k[pos] = base + np.float32(0.1) * rng.standard_normal((pos.size, d), dtype=np.float32)
        planted[heads[0]] = pos
    elif s.planted in ("per_head", "per_group"):
        # Planted logit L = sqrt(2 ln n) + 1 at beta = 1: one unit above the expected bulk maximum.
        L = math.sqrt(2.0 * math.log(n)) + 1.0
        m_total = s.n_planted if s.planted == "per_group" else s.n_planted * G
        pos = _distinct(rng, 1, cand_hi, m_total)
        order = rng.permutation(m_total)          # which planted slot lands where
        noise = rng.standard_normal((m_total, d), dtype=np.float32)
        for i in range(m_total):
            h_local = i % G
            qh = q[h_local, 0].astype(np.float64)
            c = L * math.sqrt(d) / float(np.linalg.norm(qh))
            j = pos[order[i]]
            k[j] = (c * _unit(qh).astype(np.float64)).astype(np.float32) + np.float32(0.1) * noise[i]
            planted.setdefault(heads[h_local], []).append(int(j))
        planted = {h: np.sort(np.array(p)) for h, p in planted.items()}
    elif s.planted == "per_row":
        # Plant through Q: row p gains 8 * sum of the unit vectors of m random earlier keys that are
        # outside its anchor and window, so those keys score high for that row only.
        kn = (k / np.linalg.norm(k.astype(np.float64), axis=1, keepdims=True)).astype(np.float32)
        rows = np.arange(s.W + s.n_planted, n)
        picks = np.empty((rows.size, s.n_planted), dtype=np.int64)
        for r, p in enumerate(rows):
            picks[r] = _distinct(rng, 1, p - s.W, s.n_planted)
        q[0, rows] += np.float32(8.0) * kn[picks].sum(axis=1)
        planted[heads[0]] = (rows, picks)
    elif s.planted != "none":
        raise ValueError(s.planted)

    if s.dtype == "bf16":
        q = bf16_bits_to_f32(f32_to_bf16_bits(q))
        k = bf16_bits_to_f32(f32_to_bf16_bits(k))
        v = bf16_bits_to_f32(f32_to_bf16_bits(v))
    return q, k, v, planted


@dataclass
class Workload:
    spec: WorkloadSpec
    trial: int
    q: np.ndarray        # (B, Hq, n_q, d) storage dtype: float32, or uint16 bf16 bits
    k: np.ndarray        # (B, Hkv, n_ctx, d)
    v: np.ndarray        # (B, Hkv, n_ctx, d)
    planted: dict = field(default_factory=dict)   # (b, h) -> positions

    def f32(self, name: str) -> np.ndarray:
        """Exact float32 values of q, k or v."""
        return to_f32(getattr(self, name), self.spec.dtype)


def make_workload(cfg: int, trial: int = 0, threads: int = 8, **overrides) -> Workload:
    """Generate every group of a workload (groups in parallel threads; numpy drops the GIL)."""
    s = spec(cfg, **overrides)
    store = np.uint16 if s.dtype == "bf16" else np.float32
    q = np.empty((s.B, s.Hq, s.n_q, s.d), dtype=store)
    k = np.empty((s.B, s.Hkv, s.n_ctx, s.d), dtype=store)
    v = np.empty((s.B, s.Hkv, s.n_ctx, s.d), dtype=store)
    planted: dict = {}

    def one(bg):
        b, g = bg
        qg, kg, vg, pl = gen_group(s, trial, b, g)
        conv = f32_to_bf16_bits if s.dtype == "bf16" else (lambda x: x)
        q[b, g * s.G:(g + 1) * s.G] = conv(qg)
        k[b, g] = conv(kg)
        v[b, g] = conv(vg)
        return b, pl

    groups = [(b, g) for b in range(s.B) for g in range(s.Hkv)]
    with ThreadPoolExecutor(max(1, min(threads, len(groups)))) as ex:
        for b, pl in ex.map(one, groups):
            for h, pos in pl.items():
                planted[(b, h)] = pos
    return Workload(s, trial, q, k, v, planted)
