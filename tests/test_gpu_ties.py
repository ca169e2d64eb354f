"""Ties of the GPU assignment go to the lower cluster id, for every score sign.

Each key joins the centroid of largest similarity ("ClusterKV: Manipulating
LLM KV Cache in Semantic Space for Recallable Compression", section
语义空间中的聚类, Fig. 4); equal scores go to the lower cluster id. The
initial centroids are the keys at n_sink + s c, so making those keys equal in
pairs makes every centroid tie exactly with its partner in the first
assignment, under the cosine, the inner product and L2 alike. Every key is
drawn around a common direction u, with either sign, so that its best score
is positive for half of them and negative (cosine and inner product) for the
others. Whatever pair a key's best score belongs to, the label must be the
pair's lower id: that holds for every token, with no margin exclusion. Where
the best pair beats every other centroid by the margin rule, the label must
also be the oracle's.

The pairs sit at every distance the kernel distinguishes: the same lane's
rows, another lane group of the same M tile, another M tile, another argmax
group and another LDS round (C = 600 holds two rounds); the small-window
kernel (C <= 16) and the fp32 kernel are covered too (its eight cluster
groups: pairs (0, 1) and (2, 6) sit in different groups, (3, 19) in one).
"""
import numpy as np
import pytest

import oracle
import sparse_decode_attention_ckv_amd as ck
import synth
from tests.gpu_helpers import (ASSIGN_MARGIN, CK_METRIC, gpu_cluster, margin_threshold, say,
                               to_dev)

D = 128
N_SINK = 16
METRICS = {"cosine": oracle.COSINE, "inner_product": oracle.INNER_PRODUCT, "l2": oracle.L2}


def _pairs(C, rng):
    """Partner of every cluster id (an involution without fixed points for
    even C): hand-placed pairs at the kernel's distances, the rest paired at
    random."""
    fixed = [(0, 1), (2, 6), (3, 19), (8, 136), (9, 521), (40, 599), (100, 101), (130, 515)]
    fixed = [(a, b) for a, b in fixed if b < C]
    used = {x for p in fixed for x in p}
    rest = rng.permutation([c for c in range(C) if c not in used])
    pairs = fixed + [(int(rest[2 * j]), int(rest[2 * j + 1])) for j in range(len(rest) // 2)]
    partner = np.arange(C)
    for a, b in pairs:
        partner[a], partner[b] = b, a
    return partner


def _keys(H, Lp, C, dtype, seed):
    """Keys [H][n_sink + Lp][d] with the initial centroid rows equal in pairs.
    Returns (storage, exact fp64 values, partner)."""
    rng = np.random.default_rng(seed)
    L = N_SINK + Lp
    partner = _pairs(C, rng)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    sign = np.where(rng.random((H, L, 1)) < 0.5, 1.0, -1.0)
    K = sign * (8.0 * u + 0.5 * rng.standard_normal((H, L, D)))
    K[:, :, 7] *= 3.0                                       # an outlier channel
    s = Lp // C
    pos = N_SINK + s * np.arange(C)
    # seeds of the centroids: positive side, so that the negative keys score
    # below zero against every centroid
    K[:, pos] = np.abs(K[:, pos] @ u)[..., None] * u + (K[:, pos] - (K[:, pos] @ u)[..., None] * u)
    for c in range(C):
        if partner[c] < c:
            K[:, pos[c]] = K[:, pos[partner[c]]]
    if dtype == "bf16":
        st = synth.bf16_bits(K)
        return st, synth.bf16_to_f32(st).astype(np.float64), partner
    st = K.astype(np.float32)
    return st, st.astype(np.float64), partner


def _scores(Kw, mu, metric, mode):
    """The scores the oracle compares (larger is better), from its operands:
    rows rounded to bf16 under MIRROR; for the cosine the unit centroids,
    and the unit keys under EXACT, or under MIRROR the keys as stored with
    each row divided by |k| (cosine units, as the oracle's margin). L2
    through the expansion |k|^2 - 2 k.m + |m|^2 (only gaps are used)."""
    rnd = (lambda x: synth.bf16_to_f32(synth.bf16_bits(x)).astype(np.float64)) \
        if mode == oracle.MIRROR else (lambda x: x)
    if metric == oracle.COSINE:
        mt = oracle.unit_rows(mu, mode=mode)
        if mode == oracle.EXACT:
            return oracle.unit_rows(Kw, mode=mode) @ mt.T
        k = rnd(Kw)
        return (k @ mt.T) / np.linalg.norm(k, axis=1)[:, None]
    m, k = rnd(mu), rnd(Kw)
    if metric == oracle.INNER_PRODUCT:
        return k @ m.T
    return 2 * k @ m.T - (k * k).sum(1)[:, None] - (m * m).sum(1)[None, :]


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(METRICS))
@pytest.mark.parametrize("H,Lp,C,dtype", [(2, 4096, 600, "bf16"), (2, 2048, 52, "bf16"),
                                          (2, 320, 8, "bf16"), (1, 2032, 26, "fp32")])
def test_assign_ties_go_to_lower_id(name, H, Lp, C, dtype):
    metric = METRICS[name]
    say(f"assignment ties: {name} {dtype} H={H} Lp={Lp} C={C}")
    st, Kf, partner = _keys(H, Lp, C, dtype, seed=C + Lp)
    Kd = to_dev(st, dtype)
    _, asg, _, _ = gpu_cluster(Kd, N_SINK, C, 1, metric=CK_METRIC[metric])
    a_g = asg.cpu().numpy()[:, N_SINK:]
    lower = np.minimum(np.arange(C), partner)
    # every label is the lower member of its pair
    assert np.array_equal(a_g, lower[a_g]), np.nonzero(a_g != lower[a_g])
    n_neg = n_cmp = 0
    mode = oracle.MIRROR if dtype == "bf16" else oracle.EXACT
    for h in range(H):
        mu0 = oracle.init_centroids(Kf[h], N_SINK, C)
        Kw = Kf[h][N_SINK:]
        a_o, _ = oracle.assign(Kf[h], N_SINK, mu0, mode=mode, metric=metric)
        a_o = a_o[N_SINK:]
        S = _scores(Kw, mu0, metric, mode)
        best = S[np.arange(len(Kw)), a_o]
        other = S.copy()
        other[np.arange(len(Kw)), a_o] = -np.inf
        other[np.arange(len(Kw)), partner[a_o]] = -np.inf
        gap = best - other.max(axis=1)
        thr = margin_threshold(metric, Kw, mu0, a_o, ASSIGN_MARGIN, mode)
        keep = gap >= thr
        assert np.array_equal(a_g[h][keep], a_o[keep]), h
        assert np.all(a_o == lower[a_o])            # the oracle's rule, for the record
        n_cmp += int(keep.sum())
        n_neg += int((best[keep] < 0).sum())
    say(f"  {n_cmp} labels compared with the oracle, {n_neg} of them with a negative best score")
    assert n_cmp > 0.5 * H * Lp
    assert n_neg > 0.2 * n_cmp


def test_tie_keys_are_what_the_test_needs():
    """CPU check of the construction: the seeds tie in pairs, and about half
    of the keys score negative against every centroid under the cosine."""
    st, Kf, partner = _keys(1, 4096, 600, "bf16", seed=7)
    mu0 = oracle.init_centroids(Kf[0], N_SINK, 600)
    assert np.array_equal(mu0, mu0[partner])
    S = _scores(Kf[0][N_SINK:], mu0, oracle.COSINE, oracle.MIRROR)
    neg = (S.max(axis=1) < 0).mean()
    assert 0.35 < neg < 0.65
