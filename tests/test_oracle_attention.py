"""Pins for the oracle's decode attention softmax(q K_S^T / sqrt(d)) V_S.

ClusterKV page, sections 'LLM inference and the KV cache' (dense decode
attention with q in R^{1 x d}, K, V in R^{L x d}) and 'Long-context inference
and KV compression' (the same over the B selected rows). Every check below
has an answer fixed by the mathematics, not by re-typing the formula.
"""
import math

import numpy as np
import pytest

import oracle

D = 128


def _rng(s):
    return np.random.default_rng(s)


def _one_head(K, V, q, idx, G=1):
    idx = np.asarray(idx, dtype=np.int32)[None]
    return oracle.attn(q, K[None], V[None], idx, [idx.shape[1]], G=G)


def test_single_token_returns_its_value():
    r = _rng(1)
    K, V = r.standard_normal((50, D)), r.standard_normal((50, D))
    q = r.standard_normal((1, D)) * 10
    o = _one_head(K, V, q, [17])
    assert np.array_equal(o[0], V[17])


def test_identical_keys_give_mean_of_selected_values():
    r = _rng(2)
    K = np.tile(r.standard_normal(D), (40, 1))
    V = r.standard_normal((40, D))
    q = r.standard_normal((1, D)) * 3
    sel = [3, 9, 11, 30, 31]
    o = _one_head(K, V, q, sel)
    np.testing.assert_allclose(o[0], V[sel].mean(axis=0), rtol=0, atol=1e-14)


def test_zero_query_gives_uniform_weights():
    r = _rng(3)
    K, V = r.standard_normal((64, D)) * 5, r.standard_normal((64, D))
    sel = list(range(0, 64, 3))
    o = _one_head(K, V, np.zeros((1, D)), sel)
    np.testing.assert_allclose(o[0], V[sel].mean(axis=0), atol=1e-14)


def test_scale_is_one_over_sqrt_d():
    # scores ln 3 and 0 after the 1/sqrt(d) scale -> weights 3/4 and 1/4
    K = np.zeros((2, D))
    K[0, 0] = 1.0
    V = np.zeros((2, D))
    V[0, :] = 1.0
    V[1, :] = -1.0
    q = np.zeros((1, D))
    q[0, 0] = math.sqrt(D) * math.log(3.0)
    o = _one_head(K, V, q, [0, 1])
    np.testing.assert_allclose(o[0], np.full(D, 0.75 - 0.25), atol=1e-14)


def test_two_tokens_logistic_closed_form():
    r = _rng(4)
    K, V = r.standard_normal((2, D)), r.standard_normal((2, D))
    q = r.standard_normal((1, D))
    o = _one_head(K, V, q, [0, 1])
    delta = float((q[0] @ (K[1] - K[0]))) / math.sqrt(D)
    w2 = 1.0 / (1.0 + math.exp(-delta))
    np.testing.assert_allclose(o[0], (1 - w2) * V[0] + w2 * V[1], atol=1e-13)


def test_large_common_shift_is_invariant():
    # adding u with q.u = 4e4 to every key shifts all scores by a constant; the
    # result must not change (and must not overflow).
    r = _rng(5)
    K, V = r.standard_normal((30, D)), r.standard_normal((30, D))
    q = r.standard_normal((1, D))
    u = q[0] / float(q[0] @ q[0]) * 4e4
    sel = [1, 4, 5, 20, 29]
    o1 = _one_head(K, V, q, sel)
    o2 = _one_head(K + u, V, q, sel)
    assert np.all(np.isfinite(o2))
    np.testing.assert_allclose(o1, o2, atol=1e-9)


def test_hardmax_limit():
    r = _rng(6)
    K, V = r.standard_normal((20, D)), r.standard_normal((20, D))
    q = r.standard_normal((1, D))
    sel = list(range(20))
    s = K @ q[0]
    o = _one_head(K, V, q * 1e4, sel)
    np.testing.assert_allclose(o[0], V[int(np.argmax(s))], atol=1e-12)


def test_permutation_and_linearity():
    r = _rng(7)
    K, V1, V2 = (r.standard_normal((40, D)) for _ in range(3))
    q = r.standard_normal((1, D)) * 2
    sel = [2, 5, 8, 13, 21, 34]
    a = _one_head(K, V1, q, sel)
    b = _one_head(K, V1, q, sel[::-1])
    np.testing.assert_allclose(a, b, atol=1e-14)
    c = _one_head(K, 2.5 * V1 - V2, q, sel)
    np.testing.assert_allclose(c, 2.5 * a - _one_head(K, V2, q, sel), atol=1e-13)


def test_gqa_query_head_maps_to_kv_head_h_div_g():
    G, H = 4, 2
    K = np.zeros((H, 8, D))
    V = np.zeros((H, 8, D))
    V[0] = 1.0
    V[1] = 7.0
    q = _rng(8).standard_normal((H * G, D))
    idx = np.tile(np.arange(8, dtype=np.int32), (H, 1))
    o = oracle.attn(q, K, V, idx, [8, 8], G=G)
    np.testing.assert_allclose(o[:G], 1.0, atol=1e-14)
    np.testing.assert_allclose(o[G:], 7.0, atol=1e-14)


def test_all_rows_selected_equals_dense_attention():
    r = _rng(9)
    H, G, L = 2, 4, 300
    K, V = r.standard_normal((H, L, D)), r.standard_normal((H, L, D))
    q = r.standard_normal((H * G, D)) * 2
    perm = np.stack([r.permutation(L) for _ in range(H)]).astype(np.int32)
    o = oracle.attn(q, K, V, perm, [L, L], G=G)
    od = oracle.dense_attn(q, K, V, G=G)
    np.testing.assert_allclose(o, od, atol=1e-13)
