"""Pins for the fp64 oracle: each checks it against something other than itself.

Kinds of pin (so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one):
  * values printed on the pages (slide 10 worked example, tests/golden/);
  * brute force over all k-subsets on tiny inputs;
  * reductions to an independent library routine (torch SDPA in float64):
    k = M gives full attention, k = 0 gives gists + tail, two-level with
    everything selected gives full attention over both levels, prefill with
    k >= |eligible| gives row-causal full attention;
  * closed forms (q = 0 -> plain mean over the attention set; constant V;
    one saturating key);
  * metamorphic relations (chunk permutation) and an independent dense-mask
    formulation that maps rows back to positions (the oracle maps positions
    to rows).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------- helpers ----

def sdpa(qg, K, V, mask, scale):
    """Independent reference: torch SDPA (float64, CPU) of g heads over masked rows."""
    q = torch.tensor(qg, dtype=torch.float64)[None, :, None, :]          # [1,g,1,D]
    k = torch.tensor(K, dtype=torch.float64)[None, None].expand(1, qg.shape[0], -1, -1)
    v = torch.tensor(V, dtype=torch.float64)[None, None].expand(1, qg.shape[0], -1, -1)
    m = torch.tensor(mask, dtype=torch.bool)[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)
    return o[0, :, 0, :].numpy()


def rand_unit(rng, g, D, N, C, M=None):
    M = N // C if M is None else M
    R = N + M
    return (rng.standard_normal((g, D)), rng.standard_normal((R, D)),
            rng.standard_normal((R, D)), M, R)


def row_kind(r, C, M):
    """Inverse map, written independently of the oracle: row -> ('gist', m) or ('raw', p)."""
    if r < M * (C + 1):
        m, s = divmod(r, C + 1)
        return ("gist", m) if s == C else ("raw", m * C + s)
    return ("raw", M * C + (r - M * (C + 1)))


# ------------------------------------------------- values from the pages ---

def test_slide10_worked_example():
    """Slide 10: scores 0.1/0.8/0.7/0.2 with k=2 select g2, g3 and unfold chunks 2, 3."""
    gold = json.load(open(os.path.join(GOLDEN, "slide10_topk.json")))
    S = gold["scores"]
    M, C, D = len(S), 2, 4
    N = M * C
    R = N + M
    K = np.zeros((R, D))
    V = np.arange(R * D, dtype=np.float64).reshape(R, D)
    for m, s in enumerate(S):
        K[m * (C + 1) + C, 0] = s          # gist key of chunk m scores exactly s
    qg = np.array([[1.0, 0.0, 0.0, 0.0]])
    r = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=gold["k"], tail=0,
                           scale=1.0)
    assert list(r["sel"] + 1) == gold["selected_gists_1based"]
    np.testing.assert_allclose(r["scores"], S, rtol=0, atol=0)
    # unfolded chunks: their raw rows are in the set; other chunks' raw rows are not
    raw_in = sorted({row_kind(x, C, M)[1] // C + 1 for x in r["rows"]
                     if row_kind(x, C, M)[0] == "raw"})
    assert raw_in == gold["unfolded_chunks_1based"]
    gists_in = sorted(row_kind(x, C, M)[1] for x in r["rows"] if row_kind(x, C, M)[0] == "gist")
    assert gists_in == list(range(M))      # every gist stays (hybrid attention)


def test_score_formula_one_hot_queries():
    """With q_h = e_{d_h} / scale, the group score of gist m is the mean of K[g_m, d_h]."""
    rng = np.random.default_rng(0)
    g, D, C, N = 3, 8, 4, 32
    _, K, V, M, R = rand_unit(rng, g, D, N, C)
    scale = 0.37
    dims = [5, 1, 6]
    qg = np.zeros((g, D))
    for h, d in enumerate(dims):
        qg[h, d] = 1.0 / scale
    r = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=2, tail=4, scale=scale)
    for m in range(M):
        want = (K[m * (C + 1) + C, 5] + K[m * (C + 1) + C, 1] + K[m * (C + 1) + C, 6]) / 3
        assert abs(r["scores"][m] - want) < 1e-12


# ------------------------------------------------------------ brute force --

@pytest.mark.parametrize("seed", range(12))
def test_topk_bruteforce_subsets(seed):
    """Selected set maximises the summed group score over all C(M, k) subsets."""
    rng = np.random.default_rng(100 + seed)
    g, D, C = 2, 6, 3
    M = int(rng.integers(1, 11))
    N = M * C
    _, K, V, M, R = rand_unit(rng, g, D, N, C, M)
    qg = rng.standard_normal((g, D))
    k = int(rng.integers(0, M + 1))
    r = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=k, tail=0)
    S = r["scores"]
    best, second = None, -math.inf
    best_val = -math.inf
    for sub in itertools.combinations(range(M), k):
        val = sum(S[list(sub)]) if sub else 0.0
        if val > best_val:
            best, second, best_val = sub, best_val, val
        elif val > second:
            second = val
    assert tuple(r["sel"]) == tuple(sorted(best))
    assert list(r["sel"]) == sorted(r["sel"])


def test_topk_ties_prefer_smaller_index_and_negative_zero():
    """q = 0 gives every score +0 or -0: the k smallest chunk ids win."""
    C, D, M = 4, 8, 9
    N = M * C
    R = N + M
    K = -np.abs(np.random.default_rng(1).standard_normal((R, D)))   # 0 * negative = -0
    V = np.random.default_rng(2).standard_normal((R, D))
    r = oracle.decode_unit(np.zeros((2, D)), K, V, n_raw=N, n_gist=M, chunk=C, topk=4, tail=0)
    assert list(r["sel"]) == [0, 1, 2, 3]


def test_equal_head_sums_tie_and_go_to_the_smaller_index():
    """Group score = mean of the heads' scaled logits: two gists whose per-head
    dot products differ but sum to the same value score exactly the same, so
    the smaller chunk id wins; a gist with a larger sum wins outright."""
    # D = 12: scale = 1/sqrt(12) is irrational, and summing the two heads'
    # separately rounded scaled logits would split this tie by one ulp
    C, D, M, g = 2, 12, 5, 2
    N = M * C
    R = N + M
    qg = np.zeros((g, D))
    qg[0, 0] = 1.0
    qg[1, 1] = 1.0
    K = np.zeros((R, D))
    gist = [m * (C + 1) + C for m in range(M)]
    K[gist[1], :2] = [5.0, 4.0]           # head dots (5, 4), sum 9
    K[gist[3], :2] = [6.0, 3.0]           # head dots (6, 3), sum 9: tie with chunk 1
    K[gist[4], :2] = [4.0, 4.0]           # sum 8
    V = np.random.default_rng(3).standard_normal((R, D))
    r1 = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=1, tail=0)
    assert list(r1["sel"]) == [1]
    assert r1["scores"][1] == r1["scores"][3]
    r2 = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=3, tail=0)
    assert list(r2["sel"]) == [1, 3, 4]


# --------------------------------------------------- library reductions ---

@pytest.mark.parametrize("C,M,r", [(4, 12, 0), (8, 5, 3), (16, 6, 16), (3, 7, 1)])
def test_k_equals_M_is_full_attention(C, M, r):
    rng = np.random.default_rng(C * 100 + M)
    g, D = 4, 16
    N = M * C + r
    R = N + M
    qg, K, V = rng.standard_normal((g, D)), rng.standard_normal((R, D)), rng.standard_normal((R, D))
    res = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=M, tail=r)
    ref = sdpa(qg, K, V, np.ones(R, bool), 1 / math.sqrt(D))
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)
    assert len(res["rows"]) == R


@pytest.mark.parametrize("T", [0, 1, 5, 16, 23])
def test_k_zero_is_gists_plus_tail(T):
    rng = np.random.default_rng(T)
    g, D, C, M = 2, 8, 4, 10
    N = M * C
    R = N + M
    qg, K, V = rng.standard_normal((g, D)), rng.standard_normal((R, D)), rng.standard_normal((R, D))
    res = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=0, tail=T, scale=0.3)
    mask = np.zeros(R, bool)
    mask[np.arange(C, R, C + 1)] = True                       # gist rows
    raw = np.setdiff1d(np.arange(R), np.arange(C, R, C + 1))  # raw rows in position order
    if T:
        mask[raw[-T:]] = True
    ref = sdpa(qg, K, V, mask, 0.3)
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)


def test_softmax_weights_sum_to_one_and_lse():
    rng = np.random.default_rng(7)
    g, D, C, M = 4, 32, 16, 40
    N = M * C
    qg, K, V = (rng.standard_normal((g, D)) * 3, rng.standard_normal((N + M, D)),
                rng.standard_normal((N + M, D)))
    res = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=5, tail=20)
    assert np.all(np.abs(res["wsum"] - 1) <= 1e-12)
    # lse against a direct log-sum-exp over the attention set (scipy routine)
    from scipy.special import logsumexp
    for h in range(g):
        lg = (K[res["rows"]] @ qg[h]) / math.sqrt(D)
        assert abs(res["lse"][h] - logsumexp(lg)) < 1e-10


# ----------------------------------------------------------- closed forms --

def test_q_zero_mean_over_attention_set_with_tail_overlap():
    """q = 0: uniform weights; set = gists + chunks 0..k-1 + tail, overlap counted once.

    M=6, C=4, N=24, k=3, T=14: the tail (positions 10..23) overlaps chunk 2.
    Rows written out by hand: gists 4,9,14,19,24,29; chunk 0 rows 0-3; chunk 1
    rows 5-8; chunk 2 rows 10-13 (positions 8..11, of which 10,11 are also tail);
    tail positions 12..23 -> rows 15-18, 20-23, 25-28.
    """
    C, M, N, k, T, D = 4, 6, 24, 3, 14, 5
    R = N + M
    V = np.random.default_rng(3).standard_normal((R, D))
    K = np.random.default_rng(4).standard_normal((R, D))
    res = oracle.decode_unit(np.zeros((1, D)), K, V, n_raw=N, n_gist=M, chunk=C, topk=k,
                             tail=T)
    rows = [4, 9, 14, 19, 24, 29, 0, 1, 2, 3, 5, 6, 7, 8, 10, 11, 12, 13,
            15, 16, 17, 18, 20, 21, 22, 23, 25, 26, 27, 28]
    assert sorted(rows) == list(res["rows"])
    assert len(rows) == M + k * C + T - 2
    np.testing.assert_allclose(res["out"][0], V[rows].mean(0), rtol=0, atol=1e-13)


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(5)
    g, D, C, M = 4, 16, 8, 20
    N = M * C
    R = N + M
    c = rng.standard_normal(D)
    V = np.tile(c, (R, 1))
    res = oracle.decode_unit(rng.standard_normal((g, D)) * 4, rng.standard_normal((R, D)), V,
                             n_raw=N, n_gist=M, chunk=C, topk=3, tail=8)
    np.testing.assert_allclose(res["out"], np.tile(c, (g, 1)), rtol=0, atol=1e-12)


def test_saturating_key_returns_its_value():
    rng = np.random.default_rng(6)
    D, C, M = 16, 4, 10
    N = M * C
    R = N + M
    K = rng.standard_normal((R, D)) * 0.1
    V = rng.standard_normal((R, D))
    q = rng.standard_normal(D)
    q /= np.linalg.norm(q)
    # row 48 (raw position 39, the newest token, in the tail) scores +40 above the rest
    K[48] = q * 40 * math.sqrt(D)
    res = oracle.decode_unit(q[None], K, V, n_raw=N, n_gist=M, chunk=C, topk=2, tail=4)
    assert 48 in res["rows"]
    np.testing.assert_allclose(res["out"][0], V[48], rtol=0, atol=50 * math.exp(-40) + 1e-15)


# --------------------------------------------- metamorphic / formulations --

def test_chunk_permutation_permutes_selection():
    rng = np.random.default_rng(8)
    g, D, C, M, T = 2, 8, 4, 12, 8          # tail = chunks 10, 11
    N = M * C
    R = N + M
    qg, K, V = rng.standard_normal((g, D)), rng.standard_normal((R, D)), rng.standard_normal((R, D))
    base = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=4, tail=T)
    perm = list(rng.permutation(10)) + [10, 11]      # move whole chunks (raw + gist)
    K2, V2 = np.empty_like(K), np.empty_like(V)
    for new, old in enumerate(perm):
        K2[new * (C + 1):(new + 1) * (C + 1)] = K[old * (C + 1):(old + 1) * (C + 1)]
        V2[new * (C + 1):(new + 1) * (C + 1)] = V[old * (C + 1):(old + 1) * (C + 1)]
    res = oracle.decode_unit(qg, K2, V2, n_raw=N, n_gist=M, chunk=C, topk=4, tail=T)
    assert sorted(perm[m] for m in res["sel"]) == list(base["sel"])
    np.testing.assert_allclose(res["out"], base["out"], rtol=0, atol=1e-13)


@pytest.mark.parametrize("C,M,r,k,T", [(4, 10, 0, 3, 6), (8, 7, 5, 2, 13), (16, 9, 16, 4, 40),
                                       (2, 15, 1, 15, 3)])
def test_gather_equals_dense_mask(C, M, r, k, T):
    """Logits over every row, masked by a row->position classification of our own."""
    rng = np.random.default_rng(C + M + r)
    g, D = 3, 8
    N = M * C + r
    R = N + M
    qg, K, V = rng.standard_normal((g, D)), rng.standard_normal((R, D)), rng.standard_normal((R, D))
    res = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=k, tail=T)
    sel = set(res["sel"].tolist())
    mask = np.zeros(R, bool)
    for x in range(R):
        kind, v = row_kind(x, C, M)
        if kind == "gist":
            mask[x] = True
        elif v >= N - T or (v // C < M and v // C in sel):
            mask[x] = True
    ref = sdpa(qg, K, V, mask, 1 / math.sqrt(D))
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)
    assert mask.sum() == len(res["rows"])


# ------------------------------------------------------------- two-level ---

def _hier_inputs(rng, g, D, C, M, G, r=0):
    N = M * C + r
    R = N + M
    M2 = M // G
    return (rng.standard_normal((g, D)), rng.standard_normal((R, D)),
            rng.standard_normal((R, D)), rng.standard_normal((M2, D)),
            rng.standard_normal((M2, D)), N, R, M2)


def test_hier_everything_selected_is_full_attention_over_both_levels():
    rng = np.random.default_rng(11)
    g, D, C, M, G = 4, 16, 4, 22, 4          # M2 = 5 groups, 2 orphan gists
    qg, K, V, K2, V2, N, R, M2 = _hier_inputs(rng, g, D, C, M, G)
    res = oracle.decode_hier_unit(qg, K, V, K2, V2, n_raw=N, n_gist=M, chunk=C, fanout=G,
                                  topk1=M, topk2=M2, tail=0)
    ref = sdpa(qg, np.concatenate([K2, K]), np.concatenate([V2, V]), np.ones(M2 + R, bool),
               1 / math.sqrt(D))
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)


def test_hier_all_groups_reduces_to_single_level_plus_level2_rows():
    rng = np.random.default_rng(12)
    g, D, C, M, G, k1, T = 2, 8, 4, 16, 4, 3, 6
    qg, K, V, K2, V2, N, R, M2 = _hier_inputs(rng, g, D, C, M, G)
    h = oracle.decode_hier_unit(qg, K, V, K2, V2, n_raw=N, n_gist=M, chunk=C, fanout=G,
                                topk1=k1, topk2=M2, tail=T)
    s = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=k1, tail=T)
    assert list(h["sel1"]) == list(s["sel"])
    mask = np.zeros(R, bool)
    mask[s["rows"]] = True
    ref = sdpa(qg, np.concatenate([K2, K]), np.concatenate([V2, V]),
               np.concatenate([np.ones(M2, bool), mask]), 1 / math.sqrt(D))
    np.testing.assert_allclose(h["out"], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_hier_coarse_to_fine_bruteforce(seed):
    """Level 2 picks the best k2 groups by brute force; level 1 the best k1 of their
    children (plus orphans); the set holds all candidates' gists."""
    rng = np.random.default_rng(200 + seed)
    g, D, C, G = 2, 6, 2, 3
    M = int(rng.integers(3, 14))
    qg, K, V, K2, V2, N, R, M2 = _hier_inputs(rng, g, D, C, M, G)
    k2 = int(rng.integers(0, M2 + 1))
    n_c = k2 * G + (M - M2 * G)
    k1 = int(rng.integers(0, n_c + 1))
    h = oracle.decode_hier_unit(qg, K, V, K2, V2, n_raw=N, n_gist=M, chunk=C, fanout=G,
                                topk1=k1, topk2=k2, tail=0)
    s2 = (K2 @ qg.T).mean(1)
    best2 = max(itertools.combinations(range(M2), k2), key=lambda s: sum(s2[list(s)]))
    assert tuple(h["sel2"]) == tuple(sorted(best2))
    cand = sorted({i * G + c for i in best2 for c in range(G)} | set(range(M2 * G, M)))
    assert list(h["cand1"]) == cand
    s1 = {m: (K[m * (C + 1) + C] @ qg.T).mean() for m in cand}
    best1 = max(itertools.combinations(cand, k1), key=lambda s: sum(s1[m] for m in s))
    assert tuple(h["sel1"]) == tuple(sorted(best1))
    gist_rows = {m * (C + 1) + C for m in cand}
    assert gist_rows <= set(h["rows"].tolist())


@pytest.mark.parametrize("gist_set", ["selected", "none"])
def test_hier_rules_with_every_group_reduce_to_single_level_rules(gist_set):
    """R20: with every group chosen and no orphan, the level-1 candidates are
    all gists, so the two-level step under a rule is the single-level step
    under that rule (no level-2 row joins the set)."""
    rng = np.random.default_rng(14)
    g, D, C, M, G, k1, T = 2, 8, 4, 16, 4, 3, 6
    qg, K, V, K2, V2, N, R, M2 = _hier_inputs(rng, g, D, C, M, G)
    h = oracle.decode_hier_unit(qg, K, V, K2, V2, n_raw=N, n_gist=M, chunk=C, fanout=G,
                                topk1=k1, topk2=M2, tail=T, gist_set=gist_set)
    s = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=k1, tail=T, gist_set=gist_set)
    assert list(h["sel1"]) == list(s["sel"])
    assert list(h["rows"]) == list(s["rows"])
    np.testing.assert_allclose(h["out"], s["out"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("gist_set", ["selected", "none"])
def test_hier_rules_attention_set_by_mask(gist_set):
    """R20 against a dense masked softmax: routing through two groups of a
    hierarchy with orphans, the set holds the chosen chunks' raw rows and the
    tail, plus (selected) the chosen chunks' gist rows; no level-2 row."""
    rng = np.random.default_rng(15)
    g, D, C, M, G, k2, k1, T = 3, 8, 4, 23, 4, 2, 3, 5     # M2 = 5, 3 orphans
    qg, K, V, K2, V2, N, R, M2 = _hier_inputs(rng, g, D, C, M, G, r=2)
    h = oracle.decode_hier_unit(qg, K, V, K2, V2, n_raw=N, n_gist=M, chunk=C, fanout=G,
                                topk1=k1, topk2=k2, tail=T, gist_set=gist_set)
    sel = set(h["sel1"].tolist())
    mask = np.zeros(R, bool)
    for x in range(R):
        kind, v = row_kind(x, C, M)
        if kind == "gist":
            mask[x] = gist_set == "selected" and v in sel
        elif v >= N - T or (v // C < M and v // C in sel):
            mask[x] = True
    ref = sdpa(qg, K, V, mask, 1 / math.sqrt(D))
    np.testing.assert_allclose(h["out"], ref, rtol=0, atol=1e-12)
    # the routing is the default rule's
    a = oracle.decode_hier_unit(qg, K, V, K2, V2, n_raw=N, n_gist=M, chunk=C, fanout=G,
                                topk1=k1, topk2=k2, tail=T)
    assert list(a["sel1"]) == list(h["sel1"]) and list(a["sel2"]) == list(h["sel2"])


def test_hier_orphan_gist_is_always_a_candidate():
    rng = np.random.default_rng(13)
    g, D, C, M, G = 1, 4, 2, 7, 3            # groups {0,1,2},{3,4,5}; orphan 6
    qg, K, V, K2, V2, N, R, M2 = _hier_inputs(rng, g, D, C, M, G)
    qg = np.array([[1.0, 0, 0, 0]])
    K2[:, 0] = [5.0, -5.0]                   # group 0 wins level 2
    K[6 * (C + 1) + C, 0] = 50.0             # orphan 6 is the best level-1 gist overall
    h = oracle.decode_hier_unit(qg, K, V, K2, V2, n_raw=N, n_gist=M, chunk=C, fanout=G,
                                topk1=1, topk2=1, tail=0, scale=1.0)
    assert list(h["sel2"]) == [0]
    assert list(h["sel1"]) == [6]
    assert list(h["cand1"]) == [0, 1, 2, 6]


# ---------------------------------------------------------------- prefill --

@pytest.mark.parametrize("k", [0, 3])
@pytest.mark.parametrize("t", [0, 3, 15, 16, 31, 47, 63, 100, 127])
def test_prefill_row_equals_decode_on_truncated_cache(t, k):
    rng = np.random.default_rng(14)
    g, D, C, W = 2, 8, 16, 24
    N = 128
    M = N // C
    R = N + M
    K, V = rng.standard_normal((R, D)), rng.standard_normal((R, D))
    qg = rng.standard_normal((g, D))
    p = oracle.prefill_query(qg, K, V, t=t, n_raw=N, n_gist=M, chunk=C, topk=k, window=W)
    Mt = t // C
    Rt = (t + 1) + Mt
    d = oracle.decode_unit(qg, K[:Rt], V[:Rt], n_raw=t + 1, n_gist=Mt, chunk=C,
                           topk=min(k, Mt), tail=min(W, t + 1))
    np.testing.assert_allclose(p["out"], d["out"], rtol=0, atol=1e-13)
    assert list(p["sel"][:len(d["sel"])]) == list(d["sel"])
    assert all(x == -1 for x in p["sel"][len(d["sel"]):])


@pytest.mark.parametrize("t", [0, 5, 16, 40, 79])
def test_prefill_all_eligible_is_row_causal_full_attention(t):
    rng = np.random.default_rng(15)
    g, D, C, N = 2, 8, 8, 80
    M = N // C
    R = N + M
    K, V, qg = rng.standard_normal((R, D)), rng.standard_normal((R, D)), rng.standard_normal((g, D))
    # window C covers the query's own, still gist-less chunk
    p = oracle.prefill_query(qg, K, V, t=t, n_raw=N, n_gist=M, chunk=C, topk=M, window=C)
    own_row = (t // C) * (C + 1) + t % C
    mask = np.arange(R) <= own_row
    ref = sdpa(qg, K, V, mask, 1 / math.sqrt(D))
    np.testing.assert_allclose(p["out"], ref, rtol=0, atol=1e-12)


def test_prefill_own_chunk_gist_is_not_eligible():
    D, C, N = 4, 4, 32
    M = N // C
    R = N + M
    K = np.zeros((R, D))
    V = np.random.default_rng(16).standard_normal((R, D))
    t = 3 * C + C - 1                        # last raw token of chunk 3
    K[3 * (C + 1) + C, 0] = 100.0            # gist of chunk 3 comes after t's row
    K[1 * (C + 1) + C, 0] = 1.0
    p = oracle.prefill_query(np.array([[1.0, 0, 0, 0]]), K, V, t=t, n_raw=N, n_gist=M, chunk=C,
                             topk=1, window=2, scale=1.0)
    assert list(p["sel"]) == [1]
    assert 3 * (C + 1) + C not in p["rows"]


def test_prefill_window_rows_literal():
    """t=10, C=4, W=3, k=0: gists 0,1 (rows 4, 9) + positions 8,9,10 (rows 10, 11, 12)."""
    D, C, N = 4, 4, 24
    M = N // C
    R = N + M
    rng = np.random.default_rng(17)
    K, V = rng.standard_normal((R, D)), rng.standard_normal((R, D))
    p = oracle.prefill_query(rng.standard_normal((1, D)), K, V, t=10, n_raw=N, n_gist=M,
                             chunk=C, topk=0, window=3)
    assert list(p["rows"]) == [4, 9, 10, 11, 12]


# ----------------------------------------- selection-rule variants (slide 17) ---

def _variant_mask(sel, C, M, N, T, R, gist_set):
    """Attention-set mask built from row kinds (independent of the oracle's
    position-to-row map): the rule's gists, raw rows of selected chunks, tail."""
    mask = np.zeros(R, bool)
    for r in range(R):
        kind, v = row_kind(r, C, M)
        if kind == "gist":
            mask[r] = gist_set == "all" or (gist_set == "selected" and v in sel)
        else:
            mask[r] = v >= N - T or (v // C < M and v // C in sel)
    return mask


@pytest.mark.parametrize("gist_set", ["selected", "none"])
@pytest.mark.parametrize("C,M,r,k,T", [(4, 12, 0, 3, 5), (8, 9, 3, 4, 3), (16, 6, 16, 2, 20), (3, 11, 1, 5, 1)])
def test_gist_set_variants_match_masked_sdpa(gist_set, C, M, r, k, T):
    rng = np.random.default_rng(C * 1000 + M * 10 + k)
    g, D = 3, 16
    N = M * C + r
    R = N + M
    qg, K, V = rng.standard_normal((g, D)), rng.standard_normal((R, D)), rng.standard_normal((R, D))
    base = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=k, tail=T)
    res = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=k, tail=T, gist_set=gist_set)
    np.testing.assert_array_equal(res["sel"], base["sel"])       # the rule changes the set, not the choice
    mask = _variant_mask(set(res["sel"].tolist()), C, M, N, T, R, gist_set)
    assert len(res["rows"]) == mask.sum()
    ref = sdpa(qg, K, V, mask, 1 / math.sqrt(D))
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["wsum"], 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("C,M,r", [(4, 12, 0), (8, 5, 3)])
def test_gist_set_with_k_equals_M(C, M, r):
    """Every chunk selected: the selected-gist rule is full attention, the
    raw-only rule is full attention over the raw rows."""
    rng = np.random.default_rng(C + M)
    g, D = 2, 8
    N = M * C + r
    R = N + M
    qg, K, V = rng.standard_normal((g, D)), rng.standard_normal((R, D)), rng.standard_normal((R, D))
    sg = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=M, tail=r, gist_set="selected")
    np.testing.assert_allclose(sg["out"], sdpa(qg, K, V, np.ones(R, bool), 1 / math.sqrt(D)), rtol=0, atol=1e-12)
    sr = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=M, tail=r, gist_set="none")
    raw = np.array([row_kind(i, C, M)[0] == "raw" for i in range(R)])
    np.testing.assert_allclose(sr["out"], sdpa(qg, K, V, raw, 1 / math.sqrt(D)), rtol=0, atol=1e-12)


def test_gist_set_k_zero_is_tail_only_and_empty_set_is_rejected():
    rng = np.random.default_rng(3)
    g, D, C, M, T = 2, 8, 4, 6, 5
    N = M * C
    R = N + M
    qg, K, V = rng.standard_normal((g, D)), rng.standard_normal((R, D)), rng.standard_normal((R, D))
    res = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=0, tail=T, gist_set="selected")
    tail = np.array([row_kind(i, C, M) == ("raw", row_kind(i, C, M)[1]) and row_kind(i, C, M)[1] >= N - T
                     for i in range(R)])
    np.testing.assert_allclose(res["out"], sdpa(qg, K, V, tail, 1 / math.sqrt(D)), rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=0, tail=0, gist_set="none")


@pytest.mark.parametrize("gist_set", ["all", "selected", "none"])
def test_topk_for_budget_is_the_largest_fitting_k(gist_set):
    """The chosen k's attention set (the oracle's own rows, tail placed so it
    overlaps no selected chunk) fits the budget and k + 1 would not; every
    chunk selected when the budget holds them all."""
    rng = np.random.default_rng(11)
    g, D, C, M, T = 2, 8, 4, 10, 6
    N = M * C
    R = N + M
    qg, K, V = rng.standard_normal((g, D)), rng.standard_normal((R, D)), rng.standard_normal((R, D))
    # planted: chunks 0.. score highest, so the selection stays clear of the tail
    for m in range(M):
        K[m * (C + 1) + C] = qg.mean(0) * (M - m)
    for budget in range(0, R + 5):
        k = oracle.topk_for_budget(budget, M, C, T, gist_set)
        if k < 0:
            assert (M if gist_set == "all" else 0) + T > budget
            continue
        if k == 0 and T == 0 and gist_set != "all":
            continue
        rows = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=k, tail=T,
                                  gist_set=gist_set)["rows"]
        assert len(rows) <= budget
        if k < M - -(-T // C):   # k + 1 chunks that stay clear of the tail: no overlap to shrink the set
            rows1 = oracle.decode_unit(qg, K, V, n_raw=N, n_gist=M, chunk=C, topk=k + 1, tail=T,
                                       gist_set=gist_set)["rows"]
            assert len(rows1) > budget
    assert oracle.topk_for_budget(10 ** 6, M, C, T, gist_set) == M


# ------------------------------------------------ gist tokens, cache rows ---

def test_cache_rows_are_appended_in_time_order():
    """Tokens in time order (x_0 .. x_{C-1}, g_0, x_C, ...) land on rows
    0, 1, 2, ... with no gap: the interleaved cache only ever grows at its end;
    the rows agree with the layout's own row kinds."""
    for C in (1, 3, 16):
        row = 0
        for p in range(5 * C + 2):
            assert oracle.cache_row(p, C, False) == row
            assert row_kind(row, C, 10 ** 6) == ("raw", p)
            row += 1
            if p % C == C - 1:
                m = p // C
                assert oracle.cache_row(m, C, True) == row
                assert row_kind(row, C, 10 ** 6) == ("gist", m)
                row += 1


@pytest.mark.parametrize("C,M,r,m", [(4, 12, 0, 0), (4, 12, 0, 7), (8, 5, 3, 4), (16, 6, 16, 6), (3, 9, 2, 9)])
def test_gist_query_is_masked_sdpa(C, M, r, m):
    """Gist causal mask: the chunk's raw rows and the earlier gists only
    (mask built from row kinds), against float64 SDPA."""
    rng = np.random.default_rng(C * 31 + M + m)
    g, D = 2, 16
    N = M * C + r
    R = N + M
    if (m + 1) * C > N:
        pytest.skip("chunk m incomplete")
    qg, K, V = rng.standard_normal((g, D)), rng.standard_normal((R, D)), rng.standard_normal((R, D))
    res = oracle.gist_query(qg, K, V, m=m, n_raw=N, n_gist=M, chunk=C)
    mask = np.array([(lambda k, v: (k == "gist" and v < m) or (k == "raw" and v // C == m))(*row_kind(i, C, M))
                     for i in range(R)])
    assert len(res["rows"]) == mask.sum() == C + m
    np.testing.assert_allclose(res["out"], sdpa(qg, K, V, mask, 1 / math.sqrt(D)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("m", [0, 1, 5, 11])
def test_gist_query_is_prefill_at_the_chunks_last_token(m):
    """Reduction: the gist token of chunk m sees what a prefill query at the
    chunk's last raw position sees with k = 0 and a window of C."""
    rng = np.random.default_rng(m)
    g, D, C, M = 4, 8, 4, 12
    N = M * C
    R = N + M
    qg, K, V = rng.standard_normal((g, D)), rng.standard_normal((R, D)), rng.standard_normal((R, D))
    a = oracle.gist_query(qg, K, V, m=m, n_raw=N, n_gist=M, chunk=C)
    b = oracle.prefill_query(qg, K, V, t=m * C + C - 1, n_raw=N, n_gist=M, chunk=C, topk=0, window=C)
    np.testing.assert_array_equal(a["rows"], b["rows"])
    np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=1e-13)


def test_gist_query_needs_a_complete_chunk_and_its_predecessors():
    rng = np.random.default_rng(0)
    C, M = 4, 3
    N = M * C + 2
    R = N + M
    qg, K, V = rng.standard_normal((1, 8)), rng.standard_normal((R, 8)), rng.standard_normal((R, 8))
    with pytest.raises(ValueError):
        oracle.gist_query(qg, K, V, m=3, n_raw=N, n_gist=M, chunk=C)   # chunk 3 has 2 of 4 tokens
    oracle.gist_query(qg, K, V, m=2, n_raw=N, n_gist=M, chunk=C)


# ---------------------------------------------------------------- L levels --

def _levels_inputs(rng, g, D, C, M, G, L, r=0):
    N = M * C + r
    R = N + M
    sizes = [M]
    for _ in range(2, L + 1):
        sizes.append(sizes[-1] // G)
    upper = [(rng.standard_normal((n, D)), rng.standard_normal((n, D))) for n in sizes[1:]]
    return rng.standard_normal((g, D)), rng.standard_normal((R, D)), rng.standard_normal((R, D)), upper, N, sizes


@pytest.mark.parametrize("seed", range(5))
def test_levels_two_is_the_two_level_decode(seed):
    """L = 2 is the two-level rule (pinned above on its own)."""
    rng = np.random.default_rng(500 + seed)
    g, D, C, G = 2, 8, 4, int(rng.integers(2, 5))
    M = int(rng.integers(G, 40))
    r = int(rng.integers(0, C + 1))
    qg, K, V, upper, N, sizes = _levels_inputs(rng, g, D, C, M, G, 2, r)
    k2 = int(rng.integers(0, sizes[1] + 1))
    k1 = int(rng.integers(0, k2 * G + (M - sizes[1] * G) + 1))
    T = int(rng.integers(r, N + 1))
    a = oracle.decode_levels_unit(qg, K, V, upper, n_raw=N, n_gist=M, chunk=C, fanout=G, topks=[k1, k2], tail=T)
    b = oracle.decode_hier_unit(qg, K, V, upper[0][0], upper[0][1], n_raw=N, n_gist=M, chunk=C, fanout=G,
                                topk1=k1, topk2=k2, tail=T)
    assert list(a["sels"][0]) == list(b["sel1"]) and list(a["sels"][1]) == list(b["sel2"])
    np.testing.assert_array_equal(a["rows"], b["rows"])
    np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=1e-13)


@pytest.mark.parametrize("gist_set", ["selected", "none"])
@pytest.mark.parametrize("seed", range(3))
def test_levels_rules_two_levels_are_the_two_level_rules(gist_set, seed):
    """R20 on L levels: L = 2 under a rule is the two-level step under it."""
    rng = np.random.default_rng(520 + seed)
    g, D, C, G = 2, 8, 4, int(rng.integers(2, 5))
    M = int(rng.integers(G, 40))
    r = int(rng.integers(0, C + 1))
    qg, K, V, upper, N, sizes = _levels_inputs(rng, g, D, C, M, G, 2, r)
    k2 = int(rng.integers(0, sizes[1] + 1))
    k1 = int(rng.integers(1, max(2, k2 * G + (M - sizes[1] * G) + 1)))
    k1 = min(k1, k2 * G + (M - sizes[1] * G))
    T = int(rng.integers(max(r, 1), N + 1))
    a = oracle.decode_levels_unit(qg, K, V, upper, n_raw=N, n_gist=M, chunk=C, fanout=G, topks=[k1, k2], tail=T,
                                  gist_set=gist_set)
    b = oracle.decode_hier_unit(qg, K, V, upper[0][0], upper[0][1], n_raw=N, n_gist=M, chunk=C, fanout=G,
                                topk1=k1, topk2=k2, tail=T, gist_set=gist_set)
    assert list(a["sels"][0]) == list(b["sel1"]) and list(a["sels"][1]) == list(b["sel2"])
    np.testing.assert_array_equal(a["rows"], b["rows"])
    np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=1e-13)


@pytest.mark.parametrize("gist_set", ["selected", "none"])
def test_levels_rules_attention_set_by_mask(gist_set):
    """R20 on four levels against a dense masked softmax over the level-1
    cache: no upper-level row, the chosen chunks' raw rows and the tail, and
    (selected) the chosen chunks' gist rows; the routing is the default
    rule's."""
    rng = np.random.default_rng(530)
    g, D, C, M, G, T = 2, 8, 4, 70, 3, 5
    qg, K, V, upper, N, sizes = _levels_inputs(rng, g, D, C, M, G, 4, r=1)
    topks = [4, 3, 2, 2]
    h = oracle.decode_levels_unit(qg, K, V, upper, n_raw=N, n_gist=M, chunk=C, fanout=G, topks=topks, tail=T,
                                  gist_set=gist_set)
    a = oracle.decode_levels_unit(qg, K, V, upper, n_raw=N, n_gist=M, chunk=C, fanout=G, topks=topks, tail=T)
    assert all(list(x) == list(y) for x, y in zip(h["sels"], a["sels"]))
    sel = set(h["sels"][0].tolist())
    R = N + M
    mask = np.zeros(R, bool)
    for x in range(R):
        kind, v = row_kind(x, C, M)
        if kind == "gist":
            mask[x] = gist_set == "selected" and v in sel
        elif v >= N - T or (v // C < M and v // C in sel):
            mask[x] = True
    ref = sdpa(qg, K, V, mask, 1 / math.sqrt(D))
    np.testing.assert_allclose(h["out"], ref, rtol=0, atol=1e-12)


def test_levels_everything_selected_is_full_attention_over_every_level():
    rng = np.random.default_rng(510)
    g, D, C, M, G, L = 2, 16, 3, 29, 3, 4      # sizes 29, 9, 3, 1: orphans at levels 1 and 2
    qg, K, V, upper, N, sizes = _levels_inputs(rng, g, D, C, M, G, L)
    topks = [sizes[l] for l in range(L)]      # every candidate at every level is every gist
    res = oracle.decode_levels_unit(qg, K, V, upper, n_raw=N, n_gist=M, chunk=C, fanout=G, topks=topks, tail=0)
    keys = np.concatenate([u[0] for u in upper[::-1]] + [K])
    vals = np.concatenate([u[1] for u in upper[::-1]] + [V])
    ref = sdpa(qg, keys, vals, np.ones(len(keys), bool), 1 / math.sqrt(D))
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(8))
def test_levels_coarse_to_fine_bruteforce_dense_masks(seed):
    """Three and four levels: at every level the best subset of the
    candidates by brute force, candidates from a dense mask over the level
    (parent chosen, or no full group above), and the attention set from those
    masks against float64 SDPA."""
    rng = np.random.default_rng(520 + seed)
    g, D, C, G = 2, 6, 2, 2
    L = 3 + seed % 2
    M = int(rng.integers(G ** (L - 1), 22))
    qg, K, V, upper, N, sizes = _levels_inputs(rng, g, D, C, M, G, L)
    keys_at = [np.array([K[m * (C + 1) + C] for m in range(M)])] + [u[0] for u in upper]
    vals_at = [np.array([V[m * (C + 1) + C] for m in range(M)])] + [u[1] for u in upper]
    # choose k per level top-down so that each is feasible
    topks, masks, chosen = [0] * L, [None] * L, [None] * L
    for l in range(L - 1, -1, -1):
        n = sizes[l]
        if l == L - 1:
            mask = np.ones(n, bool)
        else:
            par = np.arange(n) // G
            mask = (par >= sizes[l + 1]) | np.isin(par, list(chosen[l + 1]))
        ids = list(np.nonzero(mask)[0])
        k = int(rng.integers(0, len(ids) + 1))
        s = (keys_at[l] @ qg.T).mean(1)
        best = max(itertools.combinations(ids, k), key=lambda c: (sum(s[list(c)]), [-i for i in c]))
        topks[l], masks[l], chosen[l] = k, mask, set(best)
    res = oracle.decode_levels_unit(qg, K, V, upper, n_raw=N, n_gist=M, chunk=C, fanout=G, topks=topks, tail=0)
    for l in range(L):
        assert list(res["sels"][l]) == sorted(chosen[l]), f"level {l + 1}"
        assert list(res["cands"][l]) == list(np.nonzero(masks[l])[0]), f"level {l + 1}"
    # dense attention mask over [level L .. level 2 arrays, level-1 cache]
    keys = np.concatenate([keys_at[l] for l in range(L - 1, 0, -1)] + [K])
    vals = np.concatenate([vals_at[l] for l in range(L - 1, 0, -1)] + [V])
    m1 = np.zeros(len(K), bool)
    for x in range(len(K)):
        kind, v = row_kind(x, C, M)
        m1[x] = masks[0][v] if kind == "gist" else (v // C < M and v // C in chosen[0])
    mask = np.concatenate([masks[l] for l in range(L - 1, 0, -1)] + [m1])
    np.testing.assert_allclose(res["out"], sdpa(qg, keys, vals, mask, 1 / math.sqrt(D)), rtol=0, atol=1e-12)


def test_levels_middle_orphan_is_always_a_candidate():
    """A level-2 gist that no level-3 group covers is a candidate whatever
    level 3 chooses, and its children follow it down."""
    rng = np.random.default_rng(530)
    g, D, C, M, G, L = 1, 4, 2, 14, 3, 3     # sizes 14, 4, 1: level-2 gist 3 is ungrouped
    qg, K, V, upper, N, sizes = _levels_inputs(rng, g, D, C, M, G, L)
    qg = np.array([[1.0, 0, 0, 0]])
    upper[1][0][0, 0] = 5.0                   # the one level-3 group: children 0, 1, 2
    upper[0][0][:, 0] = [1.0, 0.0, 0.0, 40.0]  # orphan 3 is the best level-2 gist
    res = oracle.decode_levels_unit(qg, K, V, upper, n_raw=N, n_gist=M, chunk=C, fanout=G, topks=[1, 1, 1],
                                    tail=0, scale=1.0)
    assert list(res["cands"][1]) == [0, 1, 2, 3]
    assert list(res["sels"][1]) == [3]
    assert list(res["cands"][0]) == [9, 10, 11, 12, 13]   # children of 3, then level-1 orphans 12, 13


# ------------------------------------------------------------- paging ----

def _scatter_to_pages(rng, dense, P, C, n_pages):
    """Independent of the oracle: place a dense [R, D] cache into a pool of
    n_pages pages of P (C + 1) rows, page q of the sequence at pool page
    perm[q] (the rest of the pool random); returns (pool, block table)."""
    rpp = P * (C + 1)
    need = -(-dense.shape[0] // rpp)
    perm = rng.permutation(n_pages)[:need]
    pool = rng.standard_normal((n_pages, rpp, dense.shape[1]))
    for r in range(dense.shape[0]):
        pool[perm[r // rpp], r - (r // rpp) * rpp] = dense[r]
    return pool, [int(x) for x in perm]


@pytest.mark.parametrize("P,C,M,r", [(1, 4, 9, 3), (2, 16, 7, 0), (4, 8, 13, 8), (8, 2, 20, 1)])
def test_gather_pages_inverts_a_scatter(P, C, M, r):
    rng = np.random.default_rng(900 + P)
    R = M * C + r + M
    dense = rng.standard_normal((R, 5))
    pool, pages = _scatter_to_pages(rng, dense, P, C, 3 * (R // (P * (C + 1)) + 2))
    got = oracle.gather_pages(pool, pages, page_chunks=P, chunk=C, n_rows=R)
    np.testing.assert_array_equal(got, dense)
    # a chunk's C raw rows and its gist share one page
    for m in range(M):
        pg = {oracle.page_slot(m * (C + 1) + j, P, C)[0] for j in range(C + 1)}
        assert len(pg) == 1


@pytest.mark.parametrize("k", [0, 3, "M"])
def test_paged_decode_with_extra_rows_is_masked_sdpa(k):
    """Paged decode with extra rows: the dense-cache set (independent mask) plus
    the extra rows, as float64 SDPA; k = M is full attention over every cache
    row and the extras."""
    rng = np.random.default_rng(910)
    g, D, C, M, r, T, P = 2, 6, 4, 9, 2, 5, 2
    N = M * C + r
    qg, K, V, M, R = rand_unit(rng, g, D, N, C, M)
    kk = M if k == "M" else k
    kpool, pages = _scatter_to_pages(np.random.default_rng(1), K, P, C, 12)
    vpool, pages_v = _scatter_to_pages(np.random.default_rng(1), V, P, C, 12)
    assert pages == pages_v
    extra = [(pages[-1], P * (C + 1) - 1), (next(x for x in range(12) if x not in pages), 3)]
    res = oracle.decode_paged_unit(qg, kpool, vpool, pages, page_chunks=P, n_raw=N, n_gist=M, chunk=C, topk=kk,
                                   tail=T, extra_rows=extra)
    sel = set(res["sel"].tolist())
    mask = np.zeros(R, bool)
    for row in range(R):
        kind, x = row_kind(row, C, M)
        mask[row] = kind == "gist" or x >= N - T or (x < M * C and x // C in sel)
    xk = np.stack([kpool[pg, s] for pg, s in extra])
    xv = np.stack([vpool[pg, s] for pg, s in extra])
    keys, vals = np.concatenate([K, xk]), np.concatenate([V, xv])
    ref = sdpa(qg, keys, vals, np.concatenate([mask, np.ones(len(extra), bool)]), 1 / math.sqrt(D))
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)
    if k == "M":
        np.testing.assert_allclose(res["out"], sdpa(qg, keys, vals, np.ones(len(keys), bool), 1 / math.sqrt(D)),
                                   rtol=0, atol=1e-12)


def test_extra_rows_q_zero_closed_form():
    """q = 0: every weight is equal, so the output is the plain mean of V over
    the cache rows of the set and the extra rows."""
    rng = np.random.default_rng(920)
    g, D, C, M, T = 1, 4, 4, 6, 4
    N = M * C
    _, K, V, M, R = rand_unit(rng, g, D, N, C, M)
    xk, xv = rng.standard_normal((3, D)), rng.standard_normal((3, D))
    res = oracle.decode_unit(np.zeros((g, D)), K, V, n_raw=N, n_gist=M, chunk=C, topk=2, tail=T, extra=(xk, xv))
    # q = 0 ties every score: chunks 0 and 1; tail = chunk 5's raw rows
    rows = [m * (C + 1) + C for m in range(M)] + [m * (C + 1) + j for m in (0, 1) for j in range(C)]
    rows += [5 * (C + 1) + j for j in range(C)]
    want = (V[rows].sum(0) + xv.sum(0)) / (len(rows) + 3)
    np.testing.assert_allclose(res["out"][0], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("gist_set", ["selected", "none"])
def test_extra_rows_under_the_selection_rules_q_zero(gist_set):
    """R12 with R19: the rule only changes which gist rows join the set; the
    extra rows are attended under every rule. q = 0 makes the output the plain
    mean of V over the set."""
    rng = np.random.default_rng(921)
    g, D, C, M, T = 1, 4, 4, 6, 4
    N = M * C
    _, K, V, M, R = rand_unit(rng, g, D, N, C, M)
    xk, xv = rng.standard_normal((3, D)), rng.standard_normal((3, D))
    res = oracle.decode_unit(np.zeros((g, D)), K, V, n_raw=N, n_gist=M, chunk=C, topk=2, tail=T, extra=(xk, xv),
                             gist_set=gist_set)
    rows = [m * (C + 1) + C for m in (0, 1)] if gist_set == "selected" else []
    rows += [m * (C + 1) + j for m in (0, 1) for j in range(C)] + [5 * (C + 1) + j for j in range(C)]
    want = (V[rows].sum(0) + xv.sum(0)) / (len(rows) + 3)
    np.testing.assert_allclose(res["out"][0], want, rtol=0, atol=1e-12)


def test_documents_ending_mid_chunk_route_and_keep_their_last_tokens():
    """Two documents built apart and reused (chunk-sized pages): the first ends
    two tokens into a chunk. Its complete chunks and the second document's
    chunks form the routed sequence, its last two tokens are extra rows. With
    every chunk selected the result is full attention over every token and
    gist of both documents; with k = 1 the chosen chunk is the one whose gist
    is aligned with the query."""
    rng = np.random.default_rng(930)
    g, D, C = 2, 8, 4
    L1, L2 = 5 * C + 2, 4 * C + 3           # doc 2 is the query's own sequence (3 trailing raw rows)
    M1, M2 = L1 // C, L2 // C

    def doc(L, M):
        rows = []
        for m in range(M):
            rows += [("raw", m * C + j) for j in range(C)] + [("gist", m)]
        rows += [("raw", M * C + j) for j in range(L - M * C)]
        return rows, rng.standard_normal((len(rows), D)), rng.standard_normal((len(rows), D))

    r1, K1, V1 = doc(L1, M1)
    r2, K2, V2 = doc(L2, M2)
    n_pages = M1 + 1 + M2 + 1 + 3
    kpool = rng.standard_normal((n_pages, C + 1, D))
    vpool = rng.standard_normal((n_pages, C + 1, D))
    slots = rng.permutation(n_pages)
    def place(rows, K, V, first):
        used = []
        for i in range(0, len(rows), C + 1):
            pg = int(slots[first + len(used)])
            used.append(pg)
            for j in range(min(C + 1, len(rows) - i)):
                kpool[pg, j], vpool[pg, j] = K[i + j], V[i + j]
        return used
    p1 = place(r1, K1, V1, 0)                # M1 full chunk pages + one page with 2 raw rows
    p2 = place(r2, K2, V2, len(p1))
    pages = p1[:M1] + p2                      # the routed sequence: doc 1's chunks, then doc 2
    extra = [(p1[M1], 0), (p1[M1], 1)]        # doc 1's last two tokens
    N, M, T = M1 * C + L2, M1 + M2, 3
    qg = rng.standard_normal((g, D))
    res = oracle.decode_paged_unit(qg, kpool, vpool, pages, page_chunks=1, n_raw=N, n_gist=M, chunk=C, topk=M,
                                   tail=T, extra_rows=extra)
    keys, vals = np.concatenate([K1, K2]), np.concatenate([V1, V2])
    np.testing.assert_allclose(res["out"], sdpa(qg, keys, vals, np.ones(len(keys), bool), 1 / math.sqrt(D)),
                               rtol=0, atol=1e-12)
    # plant doc 1's chunk 3 gist along the mean query: it is the one chosen
    kpool[p1[3], C] = 50 * qg.mean(0) / np.linalg.norm(qg.mean(0))
    res1 = oracle.decode_paged_unit(qg, kpool, vpool, pages, page_chunks=1, n_raw=N, n_gist=M, chunk=C, topk=1,
                                    tail=T, extra_rows=extra)
    assert res1["sel"].tolist() == [3]
