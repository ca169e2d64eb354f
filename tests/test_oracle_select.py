"""Pins for the oracle's cluster-granular selection.

ClusterKV page, sections 'Cluster-granular selection' (score q.mu_i, sort
descending, take whole clusters until the budget B is reached) and
'Selection and indexing' (sizes, prefix sums, label-sorted indices; Fig. 8:
budget 3 equal to the 2nd prefix sum selects the top two clusters; the last
selected cluster is trimmed to the budget); 'Problem formulation' (the ideal
I_T is the top-B tokens by q.k).
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
D = 128


def _csr_from_lists(lists):
    """offsets/tokens rows for one head from explicit per-cluster lists."""
    off = [0]
    tok = []
    for t in lists:
        tok += list(t)
        off.append(len(tok))
    return np.array([off], np.int32), np.array([tok], np.int32)


def _int_mu_for_scores(scores, d=D):
    """Integer centroids whose inner product with q = e_0 is `scores`."""
    mu = np.zeros((1, len(scores), d))
    mu[0, :, 0] = scores
    q = np.zeros((1, d))
    q[0, 0] = 1.0
    return q, mu


def _brute_greedy(scores, lists, n_sink, B, pending=()):
    """Enumerate all cluster orders, keep the one that is non-increasing in
    score with ascending ids among equal scores, walk it greedily, then list
    sinks, pending and each admitted cluster's taken tokens by cluster id."""
    C = len(scores)
    chosen = None
    for perm in itertools.permutations(range(C)):
        ok = all(scores[perm[i]] > scores[perm[i + 1]] or
                 (scores[perm[i]] == scores[perm[i + 1]] and perm[i] < perm[i + 1])
                 for i in range(C - 1))
        if ok:
            assert chosen is None, "order must be unique"
            chosen = perm
    budget = B - n_sink - len(pending)
    taken = {}
    for c in chosen:
        room = budget - sum(taken.values())
        if room <= 0:
            break
        taken[c] = min(len(lists[c]), room)
    out = list(range(n_sink)) + list(pending)
    for c in sorted(taken):
        out += list(lists[c])[:taken[c]]
    return out


def test_fig8_golden():
    g = json.load(open(os.path.join(HERE, "golden", "fig8_budget3.json")))
    q, mu = _int_mu_for_scores(g["cluster_scores"])
    off, tok = _csr_from_lists(g["cluster_tokens"])
    C = len(g["cluster_scores"])
    for case in g["cases"]:
        idx, ns, sc = oracle.select(q, mu, off, tok, C, g["n_sink"], case["budget"])
        n = int(ns[0])
        assert list(idx[0, :n]) == case["idx"]
        assert np.all(idx[0, n:] == -1)
        order = list(np.lexsort((np.arange(C), -sc[0])))
        assert order == case["rank_order"]
        sizes = [len(g["cluster_tokens"][c]) for c in order]
        assert list(np.cumsum(sizes)) == case["prefix_sums"]


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_greedy_order(seed):
    r = np.random.default_rng(seed)
    C = int(r.integers(1, 7))
    n_sink = int(r.integers(0, 4))
    sizes = r.integers(0, 6, size=C)
    Lp = int(sizes.sum())
    perm = r.permutation(Lp) + n_sink
    lists, p = [], 0
    for s in sizes:
        lists.append(sorted(perm[p:p + s]))
        p += s
    # small integer scores, with ties on purpose
    scores = [int(x) for x in r.integers(-3, 4, size=C)]
    q, mu = _int_mu_for_scores(scores)
    # spread the integer score over several channels so the association of
    # the fp64 sum is exercised (all partial sums stay exact integers)
    mu[0, :, 5] = r.integers(-2, 3, size=C)
    q[0, 5] = 3.0
    scores = [scores[c] + 3 * int(mu[0, c, 5]) for c in range(C)]
    off, tok = _csr_from_lists(lists)
    B = n_sink + int(r.integers(0, Lp + 3))
    idx, ns, _ = oracle.select(q, mu, off, tok, C, n_sink, B)
    want = _brute_greedy(scores, lists, n_sink, B)
    assert list(idx[0, :ns[0]]) == want


def test_every_token_its_own_cluster_is_exact_topk():
    # C = L': selection must equal the ideal I_T = top-B' tokens by q.k
    r = np.random.default_rng(11)
    n_sink, Lp, Bp = 16, 300, 57
    K = r.integers(-4, 5, size=(n_sink + Lp, D)).astype(np.float64)
    q = r.integers(-3, 4, size=(1, D)).astype(np.float64)
    mu = K[None, n_sink:]
    off = np.arange(Lp + 1, dtype=np.int32)[None]
    tok = (np.arange(Lp, dtype=np.int32) + n_sink)[None]
    idx, ns, _ = oracle.select(q, mu, off, tok, Lp, n_sink, n_sink + Bp)
    s = (K[n_sink:].astype(np.int64) @ q[0].astype(np.int64))  # exact
    top = np.lexsort((np.arange(Lp), -s))[:Bp] + n_sink          # ties -> lower
    assert list(idx[0, :n_sink]) == list(range(n_sink))
    assert list(idx[0, n_sink:ns[0]]) == sorted(top)              # cluster id = position


def test_single_cluster_takes_first_positions():
    n_sink, Lp, B = 16, 200, 64
    off = np.array([[0, Lp]], np.int32)
    tok = (np.arange(Lp, dtype=np.int32) + n_sink)[None]
    q = np.ones((1, D))
    mu = np.ones((1, 1, D))
    idx, ns, _ = oracle.select(q, mu, off, tok, 1, n_sink, B)
    assert list(idx[0]) == list(range(B))


def test_budget_equal_sinks_and_budget_above_length():
    r = np.random.default_rng(12)
    n_sink, C, Lp = 16, 9, 120
    a = r.integers(0, C, size=Lp)
    lists = [list(np.nonzero(a == c)[0] + n_sink) for c in range(C)]
    off, tok = _csr_from_lists(lists)
    q = r.standard_normal((1, D))
    mu = r.standard_normal((1, C, D))
    idx, ns, _ = oracle.select(q, mu, off, tok, C, n_sink, n_sink)
    assert list(idx[0]) == list(range(n_sink))
    idx, ns, _ = oracle.select(q, mu, off, tok, C, n_sink, n_sink + Lp + 40)
    assert ns[0] == n_sink + Lp
    assert sorted(idx[0, :ns[0]]) == list(range(n_sink + Lp))
    assert np.all(idx[0, ns[0]:] == -1)
    with pytest.raises(ValueError):
        oracle.select(q, mu, off, tok, C, n_sink, n_sink - 1)


def test_pending_tokens_always_selected_and_counted():
    lists = [[16, 18], [17, 19, 20], [21]]
    off, tok = _csr_from_lists(lists)
    q, mu = _int_mu_for_scores([1, 3, 2])
    idx, ns, _ = oracle.select(q, mu, off, tok, 3, 16, 16 + 3 + 4,
                               pending_begin=22, n_pending=3)
    # ranks: cluster 1 (3 tokens), cluster 2 (1 token); emitted by cluster id
    want = list(range(16)) + [22, 23, 24] + [17, 19, 20, 21]
    assert list(idx[0, :ns[0]]) == want


def test_gqa_scores_with_sum_of_group_queries():
    r = np.random.default_rng(13)
    G, C, n_sink, Lp = 4, 12, 16, 240
    a = r.integers(0, C, size=Lp)
    lists = [list(np.nonzero(a == c)[0] + n_sink) for c in range(C)]
    off, tok = _csr_from_lists(lists)
    qs = r.integers(-5, 6, size=(G, D)).astype(np.float64)
    mu = r.integers(-5, 6, size=(1, C, D)).astype(np.float64)
    i1, n1, s1 = oracle.select(qs, mu, off, tok, C, n_sink, 100, G=G)
    i2, n2, s2 = oracle.select(qs.sum(0, keepdims=True), mu, off, tok, C, n_sink, 100)
    assert np.array_equal(i1, i2) and np.array_equal(s1, s2)
    # and the score is the exact integer inner product with the summed query
    exact = (mu[0].astype(np.int64) @ qs.sum(0).astype(np.int64))
    assert np.array_equal(s1[0], exact.astype(np.float64))


def test_score_within_fp64_error_bound_of_exact_dot():
    r = np.random.default_rng(14)
    q = r.standard_normal((1, D)) * 5
    mu = r.standard_normal((1, 20, D)) * 3
    off = np.arange(21, dtype=np.int32)[None]
    tok = np.arange(20, dtype=np.int32)[None]
    _, _, sc = oracle.select(q, mu, off, tok, 20, 0, 5)
    for c in range(20):
        exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q[0], mu[0, c]))
        bound = 130 * 2.0 ** -53 * float(np.abs(q[0] * mu[0, c]).sum())
        assert abs(float(exact) - sc[0, c]) <= bound
