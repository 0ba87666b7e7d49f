"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Source pages: "The Condensate Theorem: Transformers are O(n), Not O(n^2)" (gist.science explainers
of arXiv 2602.06317). The set definition is in the zh page's technical summary §3; the exactness
claim in its §2; the 97-position example in the fr page's popular explainer.

Each check compares the oracle with something other than itself: hand-derived sets, brute-force
rank counting and subset enumeration, exact rational arithmetic, textbook dense and sink+window
attention written with numpy matrix routines, closed forms and exact scalings. The mutation tests
at the end plant plausible mistakes in copies of the oracle and show that these checks catch them.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, gen_group, make_workload, spec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- reference checks
# Each check takes the functions under test, so the mutation tests can feed them planted mistakes.

def rank_count_topk(s, cand, k):
    """Top-k members by brute-force rank counting: j is in the top-k iff fewer than k candidates
    outrank it (higher score, or equal score at a lower position)."""
    sc = s[cand]
    higher = (sc[None, :] > sc[:, None]) | ((sc[None, :] == sc[:, None]) & (cand[None, :] < cand[:, None]))
    rank = higher.sum(axis=1)
    return np.sort(cand[rank < k])


def candidates(n, p, W, causal):
    vis_hi = p if causal else n - 1
    w_lo = max(0, p - W + 1)
    j = np.arange(vis_hi + 1)
    return j[(j != 0) & ~((j >= w_lo) & (j <= p))]


def check_invariants(set_fn, s, p, W, k, causal):
    n = s.shape[0]
    C, T = set_fn(s, p, W, k, causal)
    vis_hi = p if causal else n - 1
    w_lo = max(0, p - W + 1)
    window = np.arange(w_lo, p + 1)
    cand = candidates(n, p, W, causal)
    assert np.all(np.diff(C) > 0), "set not strictly ascending"
    assert C[0] == 0, "anchor missing"
    assert np.isin(window, C).all(), "window not inside the set"
    assert C[-1] <= vis_hi and C[0] >= 0, "set outside the visible keys"
    assert not np.isin(T, np.concatenate([[0], window])).any(), "top-k overlaps anchor or window"
    expect = len(np.union1d([0], window)) + min(k, cand.size)
    assert C.size == expect
    if causal:
        assert C.size == min(p + 1, 1 + W + k)
    np.testing.assert_array_equal(np.sort(T), rank_count_topk(s, cand, k))


def textbook_dense(q, K, V, p, scale, causal=True):
    """Softmax attention written with numpy matrix routines (BLAS dot, vectorised exp/sum)."""
    vis = p + 1 if causal else K.shape[0]
    logits = scale * (K[:vis].astype(np.float64) @ q.astype(np.float64))
    w = np.exp(logits - logits.max())
    return (w @ V[:vis].astype(np.float64)) / w.sum()


def textbook_sink_window(q, K, V, p, W, scale):
    """Attention under a mask keeping position 0 and the W most recent positions (the
    sink + sliding-window pattern the pages contrast with, zh technical summary §1)."""
    n = K.shape[0]
    j = np.arange(n)
    keep = (j == 0) | ((j > p - W) & (j <= p))
    logits = np.where(keep, scale * (K.astype(np.float64) @ q.astype(np.float64)), -np.inf)
    w = np.exp(logits - logits[keep].max())
    return (w @ V.astype(np.float64)) / w.sum()


def rand_case(rng, n, d, ties=False):
    if ties:
        q = rng.integers(-2, 3, size=d).astype(np.float32)
        K = rng.integers(-2, 3, size=(n, d)).astype(np.float32)
    else:
        q = rng.standard_normal(d).astype(np.float32)
        K = rng.standard_normal((n, d)).astype(np.float32)
    V = rng.standard_normal((n, d)).astype(np.float32)
    return q, K, V


# ----------------------------------------------------------------------------- golden fixtures

def test_golden_set_size_97():
    g = json.load(open(os.path.join(GOLDEN, "set_size_97.json")))
    rng = np.random.default_rng(97)
    q, K, V = rand_case(rng, g["n"], 16)
    s = oracle.canonical_scores(q, K)
    C, T = oracle.condensate_set(s, g["n"] - 1, g["W"], g["k"])
    assert C.size == g["expected_count"] == 97
    o, C2, _ = oracle.attend(q, K, V, g["n"] - 1, g["W"], g["k"], 0.25)
    np.testing.assert_array_equal(C, C2)


def check_hand_sets(score_fn, set_fn):
    g = json.load(open(os.path.join(GOLDEN, "hand_sets.json")))
    q = np.array(g["q"], dtype=np.float32)
    K = np.array(g["keys"], dtype=np.float32)
    s = score_fn(q, K)
    np.testing.assert_array_equal(s, [9, 5, 1, 7, 2, 7, 3, 4, 0, 6])
    for c in g["cases"]:
        C, _ = set_fn(s, c["p"], c["W"], c["k"], c["causal"])
        assert C.tolist() == c["C"], c


def test_hand_sets():
    check_hand_sets(oracle.canonical_scores, oracle.condensate_set)


# ----------------------------------------------------------------------------- set structure

def check_set_structure(set_fn, seed=0):
    rng = np.random.default_rng(seed)
    for trial in range(60):
        n = int(rng.integers(1, 300))
        ties = trial % 2 == 0
        q, K, _ = rand_case(rng, n, 8, ties=ties)
        s = oracle.canonical_scores(q, K)
        p = int(rng.integers(0, n))
        W = int(rng.integers(0, 40))
        k = int(rng.integers(0, 40))
        causal = bool(rng.integers(0, 2))
        check_invariants(set_fn, s, p, W, k, causal)


def test_set_invariants_and_rank_count():
    check_set_structure(oracle.condensate_set)


@pytest.mark.parametrize("cfg", [1, 2])
def test_rank_count_at_config_sizes(cfg):
    """Brute-force rank counting over every candidate at the tiny (n=1024) and GPT-2-small
    (n=4096) decode sizes, on the config's own inputs."""
    w = make_workload(cfg)
    s_ = w.spec
    K = w.f32("k")
    q = w.f32("q")
    for h in range(min(s_.Hq, 3)):
        s = oracle.canonical_scores(q[0, h, 0], K[0, h // s_.G])
        check_invariants(oracle.condensate_set, s, s_.n_ctx - 1, s_.W, s_.k, True)


def check_subset_enumeration(set_fn, seed=1):
    """n <= 10: among all subsets of the candidates of the right size exactly one dominates
    (every member outranks every non-member) and it is the oracle's top-k."""
    rng = np.random.default_rng(seed)
    for trial in range(40):
        n = int(rng.integers(2, 11))
        s = rng.integers(-3, 4, size=n).astype(np.float64)   # many ties on purpose
        p = int(rng.integers(0, n))
        causal = bool(rng.integers(0, 2))
        for W in range(0, n + 1):
            for k in range(0, n + 1):
                cand = candidates(n, p, W, causal)
                m = min(k, cand.size)
                dominating = []
                for S in itertools.combinations(cand.tolist(), m):
                    Sset = set(S)
                    rest = [j for j in cand.tolist() if j not in Sset]
                    if all(s[i] > s[j] or (s[i] == s[j] and i < j) for i in S for j in rest):
                        dominating.append(sorted(S))
                assert len(dominating) == 1
                _, T = set_fn(s, p, W, k, causal)
                assert sorted(T.tolist()) == dominating[0]


def test_subset_enumeration():
    check_subset_enumeration(oracle.condensate_set)


# ----------------------------------------------------------------------------- scores

def test_scores_exact_rational_bf16():
    """For bf16 data each product is exact and, on N(0,1)-scale data, so is every float64 partial
    sum: the canonical score equals the exact rational dot product."""
    s_ = spec(4, n_ctx=4096, B=1)
    q, K, _, _ = gen_group(s_, 0, 0, 0)
    rng = np.random.default_rng(5)
    js = rng.choice(K.shape[0], size=300, replace=False)
    js = np.concatenate([[0], js])          # the anchor key too
    for h in range(q.shape[0]):
        s = oracle.canonical_scores(q[h, 0], K[js])
        qf = [Fraction(float(x)) for x in q[h, 0]]
        for i, j in enumerate(js):
            exact = sum((qf[t] * Fraction(float(K[j, t])) for t in range(K.shape[1])), Fraction(0))
            assert Fraction(float(s[i])) == exact


def test_scores_fp32_error_bound():
    """fp32 data: the float64 sum is within (d-1) * 2^-53 * sum|q_t k_t| of the exact value."""
    rng = np.random.default_rng(6)
    q, K, _ = rand_case(rng, 200, 64)
    s = oracle.canonical_scores(q, K)
    qf = [Fraction(float(x)) for x in q]
    for j in range(K.shape[0]):
        exact = sum((qf[t] * Fraction(float(K[j, t])) for t in range(64)), Fraction(0))
        mag = sum(abs(float(q[t]) * float(K[j, t])) for t in range(64))
        assert abs(float(Fraction(float(s[j])) - exact)) <= 63 * 2.0 ** -53 * mag * (1 + 1e-9)


def test_scores_gqa_multihead_matches_single():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((4, 32)).astype(np.float32)
    K = rng.standard_normal((1000, 32)).astype(np.float32)
    S = oracle.canonical_scores(q, K)
    for h in range(4):
        np.testing.assert_array_equal(S[h], oracle.canonical_scores(q[h], K))


# ----------------------------------------------------------------------------- softmax over the set

def check_dense_special_case(attend_fn, seed=2):
    """1+W+k >= p+1: the set is every visible key, so the output is plain causal attention."""
    rng = np.random.default_rng(seed)
    for trial in range(20):
        n = int(rng.integers(1, 200))
        d = int(rng.choice([8, 64]))
        q, K, V = rand_case(rng, n, d)
        p = int(rng.integers(0, n))
        W = int(rng.integers(0, p + 2))
        k = max(0, p + 1 - 1 - W) + int(rng.integers(0, 3))
        scale = float(np.float32(1.0 / math.sqrt(d)))
        o, C, _ = attend_fn(q, K, V, p, W, k, scale, True)
        ref = textbook_dense(q, K, V, p, scale)
        assert C.size == p + 1
        np.testing.assert_allclose(o, ref.astype(np.float32), rtol=0, atol=2e-6 * np.abs(ref).max() + 1e-7)
        # the float64 value before rounding agrees to float64 accuracy
        s = oracle.canonical_scores(q, K)
        o64, _, _ = oracle.softmax_weighted_v(s[C], V[C], scale)
        np.testing.assert_allclose(o64, ref, rtol=1e-12, atol=1e-12)


def test_dense_special_case():
    check_dense_special_case(oracle.attend)


def check_sink_window_special_case(attend_fn, seed=3):
    """k = 0: anchor + window only, the sink + sliding-window pattern."""
    rng = np.random.default_rng(seed)
    for trial in range(20):
        n = int(rng.integers(2, 300))
        q, K, V = rand_case(rng, n, 16)
        p = n - 1
        W = int(rng.integers(0, n + 3))
        o, C, _ = attend_fn(q, K, V, p, W, 0, 0.25, True)
        ref = textbook_sink_window(q, K, V, p, W, 0.25)
        np.testing.assert_allclose(o, ref.astype(np.float32), rtol=0, atol=2e-6 * np.abs(ref).max() + 1e-7)


def test_sink_window_special_case():
    check_sink_window_special_case(oracle.attend)


def test_uniform_v_closed_form():
    """Every V row equal to u: the output is u whatever the set and the weights."""
    rng = np.random.default_rng(8)
    q, K, _ = rand_case(rng, 500, 32)
    u = rng.standard_normal(32).astype(np.float32)
    V = np.tile(u, (500, 1))
    o, _, _ = oracle.attend(q, K, V, 499, 16, 8, 0.5)
    np.testing.assert_array_equal(o, u)


def test_hard_argmax_closed_form():
    """One key far above the rest at a large scale: every other weight is below e^-100, so the
    output is that key's V row to float32 precision."""
    rng = np.random.default_rng(9)
    q, K, V = rand_case(rng, 400, 16)
    K[123] = 40.0 * q / np.linalg.norm(q)
    s = oracle.canonical_scores(q, K)
    gap = s[123] - np.max(np.delete(s, 123))
    scale = float(np.float32(100.0 / gap))
    o, C, _ = oracle.attend(q, K, V, 399, 8, 4, scale)
    assert 123 in C
    np.testing.assert_array_equal(o, V[123])


def test_power_of_two_scaling_exact():
    """V -> 2^e V scales every output bit-exactly by 2^e (no rounding changes)."""
    rng = np.random.default_rng(10)
    q, K, V = rand_case(rng, 700, 32)
    o1, C1, _ = oracle.attend(q, K, V, 699, 32, 16, 0.3)
    o2, C2, _ = oracle.attend(q, K, (V * np.float32(8.0)), 699, 32, 16, 0.3)
    np.testing.assert_array_equal(C1, C2)
    np.testing.assert_array_equal(o2, o1 * np.float32(8.0))


def test_candidate_permutation():
    """Permuting the candidate keys with their V rows (distinct scores) permutes the top-k by the
    same map and leaves the output unchanged up to summation order."""
    rng = np.random.default_rng(11)
    n, W, k = 600, 20, 10
    q, K, V = rand_case(rng, n, 16)
    p = n - 1
    perm = np.arange(n)
    inner = np.arange(1, p - W + 1)
    perm[inner] = rng.permutation(inner)
    K2, V2 = K[perm], V[perm]
    s1 = oracle.canonical_scores(q, K)
    s2 = oracle.canonical_scores(q, K2)
    C1, T1 = oracle.condensate_set(s1, p, W, k)
    C2, T2 = oracle.condensate_set(s2, p, W, k)
    np.testing.assert_array_equal(np.sort(perm[T2]), np.sort(T1))
    o1, _, _ = oracle.attend(q, K, V, p, W, k, 0.3)
    o2, _, _ = oracle.attend(q, K2, V2, p, W, k, 0.3)
    np.testing.assert_allclose(o1, o2, rtol=1e-6, atol=1e-7)


# ----------------------------------------------------------------------------- exactness claim

def exactness_check(q, K, V, p, W, k, scale, min_cert=0.99):
    s = oracle.canonical_scores(q, K)
    C, _ = oracle.condensate_set(s, p, W, k)
    o_set, _, _ = oracle.softmax_weighted_v(s[C], V[C], scale)
    o_dense = oracle.dense_attend(q, K, V, p, scale, s=s)
    rho = oracle.omitted_mass(s, C, p, scale)
    out = np.setdiff1d(np.arange(p + 1), C)
    vmax = np.abs(V[out]).max(axis=0) if out.size else np.zeros(V.shape[1])
    cert = oracle.certified_components(o_set, rho, vmax)
    ulps = oracle.ulp_distance_f32(o_set.astype(np.float32), o_dense.astype(np.float32))
    assert cert.mean() >= min_cert, (rho, cert.mean())
    assert np.all(ulps[cert] <= 1), ulps[cert].max()
    return rho, cert, ulps


def test_exactness_claim_tiny_temperature_variant():
    """Config 1 at beta = 16 (softmax_scale = 16/8 = 2): the omitted mass is below 2^-24 and the
    set output is within one float32 ulp of dense attention on every certified component."""
    s_ = spec(1, beta=16.0)
    q, K, V, _ = gen_group(s_, 0, 0, 0)
    rho, cert, ulps = exactness_check(q[0, 0], K, V, s_.n_ctx - 1, s_.W, s_.k, float(s_.softmax_scale))
    assert rho < 2.0 ** -24


@pytest.mark.parametrize("cfg,n_ctx", [(4, 131072), (5, 1 << 20)])
def test_exactness_claim_gqa_groups(cfg, n_ctx):
    """The long GQA decodes at their full context length, one kv group (4 query heads): the
    beta = 16 temperature keeps the omitted mass below 2^-24 and the set output within one
    float32 ulp of dense attention (zh technical summary §2)."""
    s_ = spec(cfg, n_ctx=n_ctx)
    q, K, V, _ = gen_group(s_, 0, 0, 0)
    for h in range(s_.G):
        rho, _, _ = exactness_check(q[h, 0], K, V, s_.n_ctx - 1, s_.W, s_.k, float(s_.softmax_scale))
        assert rho < 2.0 ** -24, (h, rho)


def test_planted_recall_and_sink_mass_statistics():
    """Generator sanity on config 2: the planted keys are retrieved by the top-k (the synthetic
    stand-in for needle retrieval, zh technical summary §5), and the anchor draws a large share of
    the set's softmax mass (30-70 % on trained models per the fr technical summary §2)."""
    w = make_workload(2)
    s_ = w.spec
    q, K, V = w.f32("q"), w.f32("k"), w.f32("v")
    hit = tot = 0
    mass = []
    for h in range(s_.Hq):
        s = oracle.canonical_scores(q[0, h, 0], K[0, h])
        C, T = oracle.condensate_set(s, s_.n_ctx - 1, s_.W, s_.k)
        planted = w.planted[(0, h)]
        hit += np.isin(planted, T).sum()
        tot += planted.size
        z = float(s_.softmax_scale) * s[C]
        wgt = np.exp(z - z.max())
        mass.append(wgt[0] / wgt.sum())
    assert hit / tot >= 0.95
    assert 0.05 < np.median(mass) < 0.9


# ----------------------------------------------------------------------------- generator

def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -3.0078125, 0.0, -0.0, 1e-30], np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_determinism_and_group_independence():
    a = make_workload(2)
    b = make_workload(2, threads=1)
    for name in ("q", "k", "v"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    s_ = spec(2)
    qg, kg, vg, _ = gen_group(s_, 0, 0, 5)
    np.testing.assert_array_equal(a.k[0, 5], kg)
    c = make_workload(2, trial=1)
    assert not np.array_equal(a.k, c.k)


# ----------------------------------------------------------------------------- planted mistakes

def _set_window_excludes_query(s, p, W, k, causal=True):
    # mistake: window is the W positions before p, not ending at p
    n = s.shape[0]
    vis_hi = p if causal else n - 1
    pos = np.arange(vis_hi + 1)
    win = (pos >= max(0, p - W)) & (pos < p)
    cand = pos[(pos != 0) & ~win]
    T = cand[np.argsort(-s[cand], kind="stable")[:min(k, cand.size)]]
    return np.unique(np.concatenate([[0], pos[win], T])), T


def _set_tie_high_index(s, p, W, k, causal=True):
    # mistake: on equal scores the higher position wins
    n = s.shape[0]
    vis_hi = p if causal else n - 1
    pos = np.arange(vis_hi + 1)
    win = (pos >= max(0, p - W + 1)) & (pos <= p)
    cand = pos[(pos != 0) & ~win][::-1]
    T = cand[np.argsort(-s[cand], kind="stable")[:min(k, cand.size)]]
    return np.unique(np.concatenate([[0], pos[win], T])), T


def _set_topk_over_all(s, p, W, k, causal=True):
    # mistake: top-k drawn from every visible key, overlapping the window
    n = s.shape[0]
    vis_hi = p if causal else n - 1
    pos = np.arange(vis_hi + 1)
    win = (pos >= max(0, p - W + 1)) & (pos <= p)
    cand = pos[pos != 0]
    T = cand[np.argsort(-s[cand], kind="stable")[:min(k, cand.size)]]
    return np.unique(np.concatenate([[0], pos[win], T])), T


def _set_no_anchor(s, p, W, k, causal=True):
    C, T = oracle.condensate_set(s, p, W, k, causal)
    return (C[1:] if (C.size and C[0] == 0 and 0 not in range(max(0, p - W + 1), p + 1)) else C), T


def _scores_transposed(q, K):
    # mistake: operands swapped in the score (q_t paired with the mirrored coordinate)
    return oracle.canonical_scores(np.asarray(q)[::-1].copy(), K)


def _attend_no_max_shift_wrong_scale(q, K, V, p, W, k, scale, causal=True):
    # mistake: the softmax scale is dropped
    return oracle.attend(q, K, V, p, W, k, 1.0, causal)


def _attend_drops_last_window_row(q, K, V, p, W, k, scale, causal=True):
    o, C, s = oracle.attend(q, K, V, p, W, k, scale, causal)
    C2 = C[C != p] if C.size > 1 else C
    o2, _, _ = oracle.softmax_weighted_v(s[C2], np.asarray(V)[C2], scale)
    return o2.astype(np.float32), C, s


@pytest.mark.parametrize("mutant", [_set_window_excludes_query, _set_tie_high_index, _set_topk_over_all,
                                    _set_no_anchor])
def test_planted_set_mistakes_are_caught(mutant):
    caught = 0
    for check in (lambda: check_hand_sets(oracle.canonical_scores, mutant),
                  lambda: check_set_structure(mutant),
                  lambda: check_subset_enumeration(mutant)):
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught >= 1


def test_planted_score_mistake_is_caught():
    with pytest.raises(AssertionError):
        check_hand_sets(_scores_transposed, oracle.condensate_set)


@pytest.mark.parametrize("mutant", [_attend_no_max_shift_wrong_scale, _attend_drops_last_window_row])
def test_planted_softmax_mistakes_are_caught(mutant):
    caught = 0
    for check in (lambda: check_dense_special_case(mutant), lambda: check_sink_window_special_case(mutant)):
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught >= 1


# ----------------------------------------------------------------------------- certificate helpers

def test_omitted_mass_matches_textbook_softmax_weights():
    """rho equals the summed textbook softmax probabilities (numpy matrix route) of the visible
    positions left out of the set."""
    rng = np.random.default_rng(13)
    q, K, _ = rand_case(rng, 900, 32)
    p, W, k, scale = 850, 40, 20, 0.4
    s = oracle.canonical_scores(q, K)
    C, _ = oracle.condensate_set(s, p, W, k)
    logits = scale * (K[:p + 1].astype(np.float64) @ q.astype(np.float64))
    prob = np.exp(logits - logits.max())
    prob /= prob.sum()
    out = np.setdiff1d(np.arange(p + 1), C)
    assert abs(oracle.omitted_mass(s, C, p, scale) - prob[out].sum()) < 1e-12


def test_ulp_distance_counts_representable_floats():
    x = np.float32(1.5)
    assert oracle.ulp_distance_f32(x, x) == 0
    assert oracle.ulp_distance_f32(x, np.nextafter(x, np.float32(2))) == 1
    y = np.nextafter(np.nextafter(x, np.float32(0)), np.float32(0))
    assert oracle.ulp_distance_f32(x, y) == 2
    assert oracle.ulp_distance_f32(np.float32(0.0), np.float32(-0.0)) == 0
    tiny = np.nextafter(np.float32(0), np.float32(1))
    assert oracle.ulp_distance_f32(tiny, -tiny) == 2


def test_certificate_bound_is_sound():
    """Where a component is certified, moving the exact output by the bound keeps the float32
    roundings within one ulp (checked against the actual dense result)."""
    s_ = spec(1, beta=16.0)
    q, K, V, _ = gen_group(s_, 0, 0, 0)
    rho, cert, ulps = exactness_check(q[0, 0], K, V, s_.n_ctx - 1, s_.W, s_.k, float(s_.softmax_scale))
    assert cert.any() and np.all(ulps[cert] <= 1)


# ----------------------------------------------------------------------------- certificate bound

def test_certificate_bound_hand_example():
    """n = 6, p = 5, W = 2, k = 1, scale 1, scores by position [0, 1, 3, 2, 0, 0]: the set is
    {0, 2, 4, 5} (anchor, the best candidate 2, window 4-5) and candidates 1 and 3 are left out.
    s_k = 3, zmax = 3, Z_C = 1 + 3 e^-3 = 1.14936120510359..., so the bound is 2 e^0 / Z_C =
    1.74009701312..."""
    s = np.array([0.0, 1.0, 3.0, 2.0, 0.0, 0.0])
    assert oracle.certificate_bound(s, 5, 2, 1, 1.0) == pytest.approx(1.7400970131228157, rel=1e-15)
    # and it bounds the true omitted mass (e^-2 + e^-1) / (Z_C + e^-2 + e^-1)
    C, _ = oracle.condensate_set(s, 5, 2, 1)
    assert oracle.omitted_mass(s, C, 5, 1.0) < oracle.certificate_bound(s, 5, 2, 1, 1.0)


def test_certificate_bound_closed_form_when_omitted_tie_the_kth():
    """If every omitted candidate scores exactly s_k, the bound is n_omit e^(z_k - m) / Z_C and the
    true omitted mass is n_omit e^(z_k - m) / (Z_C + n_omit e^(z_k - m)), so rho = b / (1 + b)."""
    rng = np.random.default_rng(31)
    n, p, W, k, scale = 400, 399, 16, 8, 0.7
    s = rng.standard_normal(n)
    cand = np.arange(1, p - W + 1)
    top = rng.choice(cand, size=k, replace=False)
    s[cand] = -1.0                       # every candidate ties at -1 ...
    s[top] = 2.0 + rng.random(k)         # ... except k clearly higher ones
    s[top[np.argmin(s[top])]] = -1.0     # the k-th is tied with the omitted ones
    C, T = oracle.condensate_set(s, p, W, k)
    assert s[T].min() == -1.0
    b = oracle.certificate_bound(s, p, W, k, scale)
    rho = oracle.omitted_mass(s, C, p, scale)
    assert rho == pytest.approx(b / (1.0 + b), rel=1e-12)


def test_certificate_bound_dominates_omitted_mass():
    """Soundness on random scores, several shapes, causal and not: the bound is never below the
    true omitted mass; it is 0 with nothing left out and +inf when k = 0 leaves candidates out."""
    rng = np.random.default_rng(32)
    for trial in range(60):
        n = int(rng.integers(2, 300))
        p = int(rng.integers(0, n))
        W, k = int(rng.integers(0, 40)), int(rng.integers(0, 40))
        causal = bool(rng.integers(0, 2))
        scale = float(rng.uniform(0.05, 3.0))
        s = rng.standard_normal(n) * float(rng.uniform(0.1, 4.0))
        C, T = oracle.condensate_set(s, p, W, k, causal)
        b = oracle.certificate_bound(s, p, W, k, scale, causal)
        rho = oracle.omitted_mass(s, C, p, scale, causal)
        vis = p + 1 if causal else n
        n_cand = vis - C.size + T.size  # visible positions outside anchor and window
        if n_cand <= k:
            assert b == 0.0 and rho == 0.0
        elif k == 0:
            assert b == float("inf")
        else:
            assert b >= rho * (1 - 1e-12)


# ----------------------------------------------------------------------------- GQA shared selection

def test_group_selection_hand_example():
    """Two query heads on one kv head, d = 2, exact integer scores worked by hand. Head 0 scores
    keys 1..4 as (3, 0, 1, 2), head 1 as (0, 2, 1, 2): the group scores are (3, 2, 1, 2); with W = 1
    (window {5}) and k = 2 the shared top-k is {1, 2} (key 2 ties key 4 and is lower), so the set
    is {0, 1, 2, 5}; on their own the heads would pick {1, 4} and {2, 4}."""
    q = np.array([[[1.0, 0.0], [0.0, 1.0]]], np.float32)           # (B=1, Hq=2, d=2)
    K = np.array([[[0, 0], [3, 0], [0, 2], [1, 1], [2, 2], [0.5, 0.5]]], np.float32)[:, None]
    V = np.arange(12, dtype=np.float32).reshape(1, 1, 6, 2) / 7.0
    scale = 0.5
    out, sel, cnt = oracle.topo_attn_decode_group(q, K, V, 1, 2, scale)
    assert cnt.tolist() == [[4, 4]]
    assert sel[0, 0, :4].tolist() == sel[0, 1, :4].tolist() == [0, 1, 2, 5]
    _, own, _ = oracle.topo_attn_decode(q, K, V, 1, 2, scale)
    assert own[0, 0, :4].tolist() == [0, 1, 4, 5] and own[0, 1, :4].tolist() == [0, 2, 4, 5]
    # textbook softmax over the shared set, per head, with each head's own scores
    C = [0, 1, 2, 5]
    for h, sh in enumerate(([0, 3, 0, 0.5], [0, 0, 2, 0.5])):
        z = scale * np.array(sh)
        w = np.exp(z - z.max())
        want = (w / w.sum()) @ V[0, 0, C].astype(np.float64)
        assert np.allclose(out[0, h], want, rtol=1e-6, atol=1e-7)


def test_group_selection_reduces_to_per_head_selection():
    rng = np.random.default_rng(41)
    # one query head per kv head: the shared set is the head's own set
    q = rng.standard_normal((2, 3, 16), dtype=np.float32)
    K = rng.standard_normal((2, 3, 200, 16), dtype=np.float32)
    V = rng.standard_normal((2, 3, 200, 16), dtype=np.float32)
    a = oracle.topo_attn_decode_group(q, K, V, 8, 12, 0.25, q_pos=150)
    b = oracle.topo_attn_decode(q, K, V, 8, 12, 0.25, q_pos=150)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    # the same query for every head of a group: the same set as each head's own
    q4 = np.repeat(rng.standard_normal((1, 2, 1, 16), dtype=np.float32), 4, axis=1)  # Hq = 8, Hkv = 2
    K2 = rng.standard_normal((1, 2, 300, 16), dtype=np.float32)
    V2 = rng.standard_normal((1, 2, 300, 16), dtype=np.float32)
    qq = np.concatenate([np.repeat(q4[:, 0:1], 4, axis=1), np.repeat(q4[:, 4:5], 4, axis=1)], axis=1)
    a = oracle.topo_attn_decode_group(qq, K2, V2, 16, 20, 0.25)
    b = oracle.topo_attn_decode(qq, K2, V2, 16, 20, 0.25)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_group_selection_rank_count_on_integer_scores():
    """Small-integer vectors make every score exact: the shared top-k must be the brute-force
    rank-count top-k of the element-wise maximum of the heads' scores."""
    rng = np.random.default_rng(42)
    for trial in range(40):
        G, n, d = int(rng.integers(1, 5)), int(rng.integers(2, 80)), 4
        q = rng.integers(-2, 3, size=(1, G, d)).astype(np.float32)
        K = rng.integers(-2, 3, size=(1, 1, n, d)).astype(np.float32)
        V = rng.standard_normal((1, 1, n, d)).astype(np.float32)
        p = int(rng.integers(0, n))
        W, k = int(rng.integers(0, 10)), int(rng.integers(0, 12))
        _, sel, cnt = oracle.topo_attn_decode_group(q, K, V, W, k, 1.0, q_pos=p)
        s = np.max(K[0, 0].astype(np.int64) @ q[0].astype(np.int64).T, axis=1).astype(np.float64)
        cand = candidates(n, p, W, True)
        want = np.union1d(np.union1d([0], np.arange(max(0, p - W + 1), p + 1)), rank_count_topk(s, cand, k))
        for h in range(G):
            assert cnt[0, h] == want.size and np.array_equal(sel[0, h, :want.size], want), (trial, h)
