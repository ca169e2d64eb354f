"""Pins of the oracle's assignment distances (no GPU).

The page keeps the cosine distance for clustering and ablates it against L2
and inner-product distance ("ClusterKV: Manipulating LLM KV Cache in Semantic
Space for Recallable Compression", section 语义空间中的聚类 and the recall
experiment with Fig. 11b). The cosine assignment is pinned elsewhere; here
the other two are pinned to hand-worked cases, a library routine, closed-form
equivalences and the Lloyd invariant of L2 K-means.
"""
import numpy as np
import pytest
from scipy.cluster.vq import vq

import oracle

# three 2-D keys against three centroids, worked by hand:
#   k0 = (10, 0): cos 1 / .707 / 0;  ip 10 / 200 / 0;  dist^2 81 / 500 / 104
#   k1 = (0, 1) : cos 0 / .707 / 1;  ip 0 / 20 / 2;    dist^2 2 / 761 / 1
#   k2 = (3, 4) : cos .6 / .990 / .8; ip 3 / 140 / 8;  dist^2 20 / 545 / 13
K2 = np.array([[10.0, 0.0], [0.0, 1.0], [3.0, 4.0]])
MU2 = np.array([[1.0, 0.0], [20.0, 20.0], [0.0, 2.0]])


@pytest.mark.parametrize("mode", [oracle.EXACT, oracle.MIRROR])
def test_hand_worked_labels(mode):
    a, m = oracle.assign(K2, 0, MU2, mode=mode, metric=oracle.COSINE)
    assert a.tolist() == [0, 2, 1]
    a, m = oracle.assign(K2, 0, MU2, mode=mode, metric=oracle.INNER_PRODUCT)
    assert a.tolist() == [1, 1, 1]
    assert m.tolist() == [190.0, 18.0, 132.0]
    a, m = oracle.assign(K2, 0, MU2, mode=mode, metric=oracle.L2)
    assert a.tolist() == [0, 2, 2]
    assert m.tolist() == [23.0, 1.0, 7.0]           # squared-distance gaps


def test_sinks_and_ties():
    K = np.array([[5.0, 5.0], [1.0, 0.0], [0.0, 3.0]])
    mu = np.array([[2.0, 0.0], [2.0, 0.0], [0.0, 1.0]])      # clusters 0 and 1 coincide
    for metric in (oracle.INNER_PRODUCT, oracle.L2):
        a, m = oracle.assign(K, 1, mu, mode=oracle.EXACT, metric=metric)
        assert a[0] == -1 and np.isinf(m[0])
        assert a[1] == 0 and m[1] == 0.0                    # tie -> lower id
        assert a[2] == 2


def test_mirror_rounds_operands_to_bf16():
    # 1 + 2^-10 is not a bf16 value: it rounds to 1, so the two centroids tie
    # under MIRROR (the lower id wins) but not under EXACT
    K = np.array([[1.0, 0.0]])
    mu = np.array([[1.0, 0.0], [1.0 + 2.0 ** -10, 0.0]])
    assert oracle.assign(K, 0, mu, mode=oracle.EXACT, metric=oracle.INNER_PRODUCT)[0][0] == 1
    assert oracle.assign(K, 0, mu, mode=oracle.MIRROR, metric=oracle.INNER_PRODUCT)[0][0] == 0
    K = np.array([[1.0 + 2.0 ** -9, 0.0]])        # L2: nearer the larger one, exactly
    assert oracle.assign(K, 0, mu, mode=oracle.EXACT, metric=oracle.L2)[0][0] == 1
    assert oracle.assign(K, 0, mu, mode=oracle.MIRROR, metric=oracle.L2)[0][0] == 0


def test_l2_matches_scipy_vq():
    rng = np.random.default_rng(5)
    K = rng.normal(size=(600, 16)) * rng.uniform(0.2, 3.0, size=(600, 1))
    mu = rng.normal(size=(23, 16))
    a, m = oracle.assign(K, 0, mu, mode=oracle.EXACT, metric=oracle.L2)
    code, dist = vq(K, mu)
    keep = m > 1e-9
    assert keep.sum() > 590
    assert np.array_equal(a[keep], code[keep])
    # the squared distance of the chosen centroid is the library's
    best = np.array([np.sum((K[i] - mu[a[i]]) ** 2) for i in range(len(K))])
    assert np.allclose(best, dist ** 2, rtol=1e-12, atol=1e-12)


def test_equal_norm_centroids_make_the_three_agree():
    # |k - mu|^2 = |k|^2 + b^2 - 2<k, mu> and cos = <k, mu> / (|k| b) when
    # every |mu_c| = b: the three orders coincide
    rng = np.random.default_rng(9)
    K = rng.normal(size=(500, 32)) * rng.uniform(0.1, 10.0, size=(500, 1))
    mu = rng.normal(size=(40, 32))
    mu *= 2.5 / np.linalg.norm(mu, axis=1, keepdims=True)
    a_c, m_c = oracle.assign(K, 0, mu, mode=oracle.EXACT, metric=oracle.COSINE)
    a_i, m_i = oracle.assign(K, 0, mu, mode=oracle.EXACT, metric=oracle.INNER_PRODUCT)
    a_l, m_l = oracle.assign(K, 0, mu, mode=oracle.EXACT, metric=oracle.L2)
    keep = (m_c > 1e-9) & (m_i > 1e-9) & (m_l > 1e-9)
    assert keep.sum() > 490
    assert np.array_equal(a_i[keep], a_c[keep])
    assert np.array_equal(a_l[keep], a_c[keep])
    # and with unequal centroid norms they differ (the ablation is not void)
    mu2 = mu * rng.uniform(0.2, 5.0, size=(40, 1))
    assert not np.array_equal(oracle.assign(K, 0, mu2, mode=oracle.EXACT,
                                            metric=oracle.INNER_PRODUCT)[0],
                              oracle.assign(K, 0, mu2, mode=oracle.EXACT,
                                            metric=oracle.COSINE)[0])


def _sse(K, n_sink, a, mu):
    return sum(float(np.sum((K[i] - mu[a[i]]) ** 2)) for i in range(n_sink, len(K)))


def test_l2_lloyd_never_increases_the_squared_error():
    rng = np.random.default_rng(11)
    centers = rng.normal(size=(6, 8)) * 4
    K = centers[rng.integers(0, 6, 400)] + rng.normal(size=(400, 8))
    n_sink, C, iters = 4, 6, 8
    mu = oracle.init_centroids(K, n_sink, C)
    prev = None
    labels = []
    for _ in range(iters):
        a, _ = oracle.assign(K, n_sink, mu, mode=oracle.EXACT, metric=oracle.L2)
        e_assign = _sse(K, n_sink, a, mu)
        if prev is not None:
            assert e_assign <= prev + 1e-9
        mu = oracle.update(K, n_sink, a, mu, mode=oracle.EXACT)
        e_update = _sse(K, n_sink, a, mu)
        assert e_update <= e_assign + 1e-9
        prev = e_update
        labels.append(a)
    # the whole loop in one call gives the same partition and centroids
    out = oracle.cluster(K, n_sink, C, iters, mode=oracle.EXACT, metric=oracle.L2)
    assert np.array_equal(out["assign"], labels[-1])
    assert np.allclose(out["mu"], mu, rtol=0, atol=0)
    # every row is at its nearest centroid of the previous iteration, which
    # is how L2 K-means ends on well separated blobs
    assert out["changed"][-1] == 0


def test_cosine_default_unchanged_by_metric_argument():
    rng = np.random.default_rng(3)
    K = rng.normal(size=(300, 16))
    a0 = oracle.cluster(K, 2, 7, 4)
    a1 = oracle.cluster(K, 2, 7, 4, metric=oracle.COSINE)
    for k in ("mu", "assign", "offsets", "tokens", "changed"):
        assert np.array_equal(a0[k], a1[k])
    with pytest.raises(AssertionError):
        oracle.cluster(K, 2, 7, 4, trace=True, metric=oracle.L2)
