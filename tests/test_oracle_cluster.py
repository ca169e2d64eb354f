"""Pins for the oracle's semantic clustering and its cluster index.

ClusterKV page, section 'Clustering in semantic space' (cosine distance D,
K-means: sampled keys as initial centroids, alternate assignment to the
centroid of largest cosine similarity and update to the mean of the assigned
keys; the first 16 tokens are kept out as attention sinks; C0 = L/80;
decode tokens are clustered every m = 320 steps into C+ = 4 clusters), and
'Selection and indexing' (sizes, prefix sums, label-sorted token indices).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

D = 128


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(4000) * 10 ** r.uniform(-3, 3, 4000),
                        # exact ties between two bf16 values
                        (np.arange(1, 200) * 2.0 + 1.0) * 2.0 ** -8])
    x = x.astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_round(float(v)) for v in x])
    assert np.array_equal(got, want)


def test_objective_non_increasing_exact():
    wl = synth.workload(0)
    hd = synth.make_head(wl, 0)
    r = oracle.cluster(hd.Kf, 16, 25, 10, mode=oracle.EXACT, trace=True)
    tr = r["trace"]
    assert np.all(np.diff(tr) <= 1e-12 * tr[0]), np.diff(tr).max()
    # second workload seed, different C
    r2 = oracle.cluster(synth.make_head(wl, 0, L=700).Kf, 16, 7, 8,
                        mode=oracle.EXACT, trace=True)
    assert np.all(np.diff(r2["trace"]) <= 1e-12 * r2["trace"][0])


@pytest.mark.parametrize("mode", [oracle.EXACT, oracle.MIRROR])
def test_planted_clusters_recovered_exactly(mode):
    n_dirs, n_sink = 12, 16
    L = n_sink + n_dirs * 60
    _, Kf, z = synth.planted_head(n_dirs, L, D, n_sink, seed=5)
    r = oracle.cluster(Kf, n_sink, n_dirs, 3, mode=mode)
    # init token c comes from planted direction c, so labels must coincide
    assert np.array_equal(r["assign"][n_sink:], z[n_sink:])
    assert r["changed"][-1] == 0


def test_single_cluster_centroid_is_mean_of_non_sink_keys():
    r = np.random.default_rng(2)
    K = r.standard_normal((300, D)) * 3
    out = oracle.cluster(K, 16, 1, 2, mode=oracle.EXACT)
    assert np.all(out["assign"][16:] == 0) and np.all(out["assign"][:16] == -1)
    np.testing.assert_allclose(out["mu"][0], K[16:].mean(axis=0), atol=1e-12)


def test_every_token_own_cluster_is_fixed_point():
    r = np.random.default_rng(3)
    n_sink, Lp = 4, 60
    K = r.standard_normal((n_sink + Lp, D))
    out = oracle.cluster(K, n_sink, Lp, 3, mode=oracle.EXACT)
    assert np.array_equal(out["assign"][n_sink:], np.arange(Lp))
    np.testing.assert_array_equal(out["mu"], K[n_sink:])


def test_assignment_is_cosine_not_inner_product_or_l2():
    mu = np.zeros((2, D))
    mu[0, 0] = 1.0
    mu[1, 0] = mu[1, 1] = 10.0 / np.sqrt(2)
    k = np.zeros((1, D))
    k[0, 0], k[0, 1] = 1.0, 0.1
    # inner product would pick centroid 1 (7.8 > 1.0) and so would L2 after
    # scaling the key up; cosine picks centroid 0 (0.995 > 0.774)
    for scale in (1.0, 7.0, 70.0):
        a, m = oracle.assign(k * scale, 0, mu, mode=oracle.EXACT)
        assert a[0] == 0
        cos0 = 1.0 / np.hypot(1.0, 0.1)
        cos1 = 1.1 / np.sqrt(2) / np.hypot(1.0, 0.1)
        assert abs(m[0] - (cos0 - cos1)) < 1e-14


def test_update_is_mean_of_raw_keys_not_of_unit_keys():
    K = np.zeros((3, D))
    K[0, 0] = 1.0            # sink
    K[1, 0] = 10.0
    K[2, 1] = 1.0
    out = oracle.cluster(K, 1, 1, 1, mode=oracle.EXACT)
    want = np.zeros(D)
    want[0], want[1] = 5.0, 0.5          # unit-key mean would be (0.5, 0.5)
    np.testing.assert_array_equal(out["mu"][0], want)


def test_ties_go_to_lower_id_and_empty_cluster_keeps_centroid():
    r = np.random.default_rng(4)
    n_sink, Lp, C = 2, 40, 4
    K = r.standard_normal((n_sink + Lp, D))
    s = Lp // C
    # clusters 1 and 3 start from copies of the key that seeds cluster 0
    K[n_sink + s] = K[n_sink]
    K[n_sink + 3 * s] = 2.0 * K[n_sink]
    out = oracle.cluster(K, n_sink, C, 1, mode=oracle.EXACT)
    a = out["assign"][n_sink:]
    assert not np.any(a == 1) and not np.any(a == 3)
    np.testing.assert_array_equal(out["mu"][1], K[n_sink + s])
    np.testing.assert_array_equal(out["mu"][3], K[n_sink + 3 * s])
    assert out["offsets"][1] == out["offsets"][2]
    assert out["offsets"][3] == out["offsets"][4]


def test_csr_structure_and_stable_sort():
    wl = synth.workload(0)
    hd = synth.make_head(wl, 0)
    base = 1000
    out = oracle.cluster(hd.Kf, 16, 25, 4, mode=oracle.MIRROR, token_base=base)
    a, off, tok = out["assign"], out["offsets"], out["tokens"]
    Lp = wl.L - 16
    assert off[0] == 0 and off[-1] == Lp and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.sort(tok), np.arange(16, wl.L) + base)
    for c in range(25):
        seg = tok[off[c]:off[c + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(a[seg - base] == c)
    want = np.argsort(a[16:], kind="stable") + 16 + base
    assert np.array_equal(tok, want)
    assert np.array_equal(np.diff(off), np.bincount(a[16:], minlength=25))


def test_fixed_point_repeats_exactly():
    n_dirs, n_sink = 6, 16
    L = n_sink + n_dirs * 40
    _, Kf, _ = synth.planted_head(n_dirs, L, D, n_sink, seed=9)
    r3 = oracle.cluster(Kf, n_sink, n_dirs, 3, mode=oracle.MIRROR)
    r9 = oracle.cluster(Kf, n_sink, n_dirs, 9, mode=oracle.MIRROR)
    assert r9["changed"][-1] == 0
    assert np.array_equal(r3["mu"], r9["mu"])
    assert np.array_equal(r3["tokens"], r9["tokens"])


def _bf16_of_fp32_of_quotient(X):
    """Independent path for the MIRROR operands: numpy's sequential fp64
    sum of the exact squares (x_j^2 is exact in fp64 for fp32/bf16 inputs,
    so this is the definition's fp64 chain), numpy's sqrt and division,
    numpy's fp64 -> fp32 cast and torch's fp32 -> bf16 cast (both round to
    nearest-even)."""
    X = np.asarray(X, dtype=np.float64)
    n = np.sqrt(np.cumsum(X * X, axis=1)[:, -1:])
    u32 = (X / n).astype(np.float32)
    return torch.from_numpy(u32).to(torch.bfloat16).double().numpy(), X / n


def test_mirror_operands_are_bf16_of_fp32_of_unit_vector():
    """Every MIRROR operand bit equals bf16(fl32(k_j / |k|)) computed by the
    independent path, on keys drawn like the workload's (bf16 storage, fp32
    storage and wide dynamic range). The sample must hold double-rounding
    cases -- where rounding the fp64 quotient straight to bf16 gives another
    value -- so that an oracle skipping the fp32 step would fail."""
    r = np.random.default_rng(6)
    wl = synth.workload(1)
    hd = synth.make_head(wl, 0, L=4096)
    X = np.concatenate([
        hd.Kf,                                                         # bf16 keys
        (r.standard_normal((2048, D)) * 20).astype(np.float32),       # fp32 keys
        (r.standard_normal((2048, D)) * 10.0 ** r.uniform(-3, 3, (2048, 1))
         ).astype(np.float32)]).astype(np.float64)
    u = oracle.unit_rows(X, mode=oracle.MIRROR)
    want, q = _bf16_of_fp32_of_quotient(X)
    assert np.array_equal(u, want)
    # fp64 -> bf16 in one rounding (nearest-even on the 8-bit significand)
    m, e = np.frexp(q)
    direct = np.ldexp(np.rint(m * 256.0) / 256.0, e)
    assert np.count_nonzero(direct != want) > 0
    # the EXACT operand is the fp64 quotient itself
    assert np.array_equal(oracle.unit_rows(X, mode=oracle.EXACT), q)


def test_mirror_operands_of_centroids_in_assignment():
    """The MIRROR cosine compares fp64 dot products of the key as stored
    (bf16, rounded here by torch) with the independently rounded unit
    centroids, and its margin is their gap divided by |k|. The label is the
    EXACT cosine's wherever the cosines are not near a tie, and the margin
    is within the rounding of the unit centroids of the exact cosine gap."""
    r = np.random.default_rng(11)
    for _ in range(20):
        k = r.standard_normal((1, D)) * 5 * 10.0 ** r.uniform(-2, 2)
        mu = r.standard_normal((2, D)) * 3
        a, m = oracle.assign(k, 0, mu, mode=oracle.MIRROR)
        kb = torch.from_numpy(k).to(torch.bfloat16).double().numpy()
        mt, mq = _bf16_of_fp32_of_quotient(mu)
        s = np.array([np.dot(kb[0], mt[c]) for c in range(2)])
        nk = np.sqrt(np.sum(kb[0] ** 2))
        assert a[0] == int(np.argmax(s))
        assert abs(m[0] - abs(s[0] - s[1]) / nk) <= 1e-15
        # each rounded unit element is within 2^-8 (relative) of the exact
        # one, so each cosine moves by at most 2^-8 |k||u| / |k| = 2^-8
        cos = np.array([np.dot(kb[0], mq[c]) / nk for c in range(2)])
        bound = 2 * 2.0 ** -8 * (1 + 2.0 ** -20)
        assert abs(m[0] - abs(cos[0] - cos[1])) <= bound
        if abs(cos[0] - cos[1]) > bound:
            assert a[0] == int(np.argmax(cos))


def test_mirror_cosine_key_scale_and_zero_key():
    """Scaling a key by a power of two scales every MIRROR score and leaves
    the labels and cosine margins unchanged; a zero key ties everywhere,
    goes to cluster 0 with margin 0."""
    r = np.random.default_rng(12)
    K = torch.from_numpy(r.standard_normal((300, D))).to(torch.bfloat16).double().numpy()
    mu = r.standard_normal((17, D))
    a1, m1 = oracle.assign(K, 0, mu, mode=oracle.MIRROR)
    for sc in (2.0 ** -20, 2.0 ** 7):
        a2, m2 = oracle.assign(K * sc, 0, mu, mode=oracle.MIRROR)
        assert np.array_equal(a1, a2)
        assert np.allclose(m1, m2, rtol=1e-12, atol=0)
    a0, m0 = oracle.assign(np.zeros((1, D)), 0, mu, mode=oracle.MIRROR)
    assert a0[0] == 0 and m0[0] == 0.0


def test_objective_closed_forms():
    """J_w = sum_i (|k_i| - <k_i, mu_a>/|mu_a|), pinned by values that hold
    whatever the data: a hand-worked 2-D case; C = L' with every token its
    own centroid gives 0; C = 1 with the mean as centroid gives
    sum |k_i| - |sum k_i|; a zero centroid contributes |k_i|; scaling the
    keys by a scales J by a, scaling a centroid leaves J unchanged."""
    # hand-worked: k = (3, 4), mu = (1, 0): |k| = 5, <k, mu>/|mu| = 3 -> 2;
    # k = (0, 2), mu = (0, -7): 2 - (-2) = 4; sinks never count
    K = np.array([[9.0, 9.0], [3.0, 4.0], [0.0, 2.0]])
    mu = np.array([[1.0, 0.0], [0.0, -7.0]])
    assert oracle.objective(K, 1, np.array([-1, 0, 1]), mu) == 6.0

    r = np.random.default_rng(12)
    n_sink, Lp = 4, 200
    Kr = r.standard_normal((n_sink + Lp, D)) * 3
    own = np.concatenate([-np.ones(n_sink, np.int32), np.arange(Lp, dtype=np.int32)])
    J_own = oracle.objective(Kr, n_sink, own, Kr[n_sink:])
    assert abs(J_own) <= 1e-12 * np.linalg.norm(Kr[n_sink:], axis=1).sum()

    one = np.concatenate([-np.ones(n_sink, np.int32), np.zeros(Lp, np.int32)])
    mean = Kr[n_sink:].mean(axis=0, keepdims=True)
    want = np.linalg.norm(Kr[n_sink:], axis=1).sum() - np.linalg.norm(Kr[n_sink:].sum(axis=0))
    got = oracle.objective(Kr, n_sink, one, mean)
    assert abs(got - want) <= 1e-10 * abs(want), (got, want)

    zero = np.zeros((1, D))
    assert abs(oracle.objective(Kr, n_sink, one, zero)
               - np.linalg.norm(Kr[n_sink:], axis=1).sum()) <= 1e-10 * Lp

    lab = np.concatenate([-np.ones(n_sink, np.int32), r.integers(0, 5, Lp).astype(np.int32)])
    mu5 = r.standard_normal((5, D))
    J = oracle.objective(Kr, n_sink, lab, mu5)
    assert abs(oracle.objective(2.5 * Kr, n_sink, lab, mu5) - 2.5 * J) <= 1e-10 * abs(J)
    assert abs(oracle.objective(Kr, n_sink, lab, mu5 * np.arange(1, 6)[:, None]) - J) \
        <= 1e-10 * abs(J)
    # the value matches the definition's terms summed independently
    km = mu5[lab[n_sink:]]
    terms = np.linalg.norm(Kr[n_sink:], axis=1) - np.einsum(
        "ij,ij->i", Kr[n_sink:], km) / np.linalg.norm(km, axis=1)
    assert abs(J - terms.sum()) <= 1e-10 * np.abs(terms).sum()


def test_objective_trace_is_the_objective_of_each_state():
    """The trace's entries are J_w of the partition after each assignment
    (against the centroids it was assigned with) and after each update
    (against the new means): recompute both from oracle.assign/update."""
    wl = synth.workload(0)
    hd = synth.make_head(wl, 0, L=600)
    C, iters, n_sink = 7, 4, 16
    r = oracle.cluster(hd.Kf, n_sink, C, iters, mode=oracle.EXACT, trace=True)
    mu = oracle.init_centroids(hd.Kf, n_sink, C)
    for t in range(iters):
        a, _ = oracle.assign(hd.Kf, n_sink, mu, mode=oracle.EXACT)
        assert r["trace"][2 * t] == oracle.objective(hd.Kf, n_sink, a, mu)
        mu = oracle.update(hd.Kf, n_sink, a, mu, mode=oracle.EXACT)
        assert r["trace"][2 * t + 1] == oracle.objective(hd.Kf, n_sink, a, mu)


def test_incremental_window_labels_and_absolute_ids():
    # decode-time increments: no sinks, C+ = 4 clusters among m = 320 tokens,
    # token ids continue after the prompt
    r = np.random.default_rng(7)
    m, Cp, base = 320, 4, 32768 + 320
    K = r.standard_normal((m, D))
    out = oracle.cluster(K, 0, Cp, 10, mode=oracle.MIRROR, token_base=base)
    assert np.all(out["assign"] >= 0)
    assert np.array_equal(np.sort(out["tokens"]), np.arange(m) + base)
    # init tokens are base + 80 c
    mu0 = oracle.init_centroids(K, 0, Cp)
    np.testing.assert_array_equal(mu0, K[[0, 80, 160, 240]])
