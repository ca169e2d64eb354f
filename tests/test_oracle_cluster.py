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


def test_mirror_operands_are_bf16_of_fp32_of_unit_vector():
    r = np.random.default_rng(6)
    X = r.standard_normal((50, D)) * 20
    u = oracle.unit_rows(X, mode=oracle.MIRROR)
    ex = X / np.linalg.norm(X, axis=1, keepdims=True)
    want = torch.from_numpy(ex.astype(np.float32)).to(torch.bfloat16).double().numpy()
    # the oracle's fp64 norm differs from numpy's only in the last bits; the
    # rounded operands agree except at a rounding boundary
    assert np.mean(u == want) > 0.999
    np.testing.assert_allclose(u, ex, atol=2 ** -8)


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
