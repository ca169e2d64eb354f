"""Clustering properties that follow from the distances themselves (GPU).

The cosine, inner-product and L2 assignments of "ClusterKV: Manipulating LLM
KV Cache in Semantic Space for Recallable Compression" (section
语义空间中的聚类, distance D, and the ablation with Fig. 11b) and the mean
update are all equivariant under scaling every key by the same factor: the
cosine does not see the factor, the inner-product and L2 scores scale by its
square, and the means scale by it. For a power of two the GPU path is
equivariant bit for bit: bf16 and fp32 values scale exactly, products and
sums of scaled values are the scaled products and sums (no value here comes
near overflow or underflow), and the cosine's per-token offset, twice the
key's norm, scales with the key. So labels and CSR must be identical and the
centroids exactly scaled.

A zero key has cosine 0 with every centroid: the oracle, scanning clusters in
id order with a strict comparison, gives it cluster 0, and so must the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import CK_METRIC, gpu_cluster, say, to_dev

pytestmark = pytest.mark.gpu

METRICS = {"cosine": oracle.COSINE, "inner_product": oracle.INNER_PRODUCT, "l2": oracle.L2}


def _keys(H, L, dtype):
    wl = synth.workload(1 if dtype == "bf16" else 0)
    K, _, _ = synth.make_kv(wl, L=L, heads=range(H)) if dtype == "bf16" else \
        synth.make_kv(wl, L=L)
    return to_dev(K, dtype)


@pytest.mark.parametrize("name", list(METRICS))
@pytest.mark.parametrize("H,L,C,dtype", [(2, 4112, 51, "bf16"), (8, 336, 4, "bf16"),
                                          (1, 2048, 25, "fp32")])
def test_power_of_two_key_scale_is_exact(name, H, L, C, dtype):
    say(f"key scale equivariance: {name} {dtype} H={H} L={L} C={C}")
    Kd = _keys(H, L, dtype)
    metric = CK_METRIC[METRICS[name]]
    c1, a1, o1, t1 = gpu_cluster(Kd, 16, C, 6, metric=metric)
    for e in (-12, 9):
        say(f"  keys x 2^{e}")
        c2, a2, o2, t2 = gpu_cluster((Kd.float() * 2.0 ** e).to(Kd.dtype), 16, C, 6,
                                     metric=metric)
        assert torch.equal(a1, a2), e
        assert torch.equal(o1, o2) and torch.equal(t1, t2), e
        assert torch.equal(c1 * 2.0 ** e, c2), e


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_zero_keys_join_cluster_zero(dtype):
    say(f"zero keys, cosine, {dtype}")
    H, L, C = 2, 2064, 24
    Kd = _keys(H, L, dtype) if dtype == "bf16" else _keys(1, L, dtype).repeat(2, 1, 1)
    Kd = Kd.clone()
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(np.arange(16, L), 200, replace=False))
    # keep the rows the initial centroids are taken from non-zero
    init = 16 + ((L - 16) // C) * np.arange(C)
    rows = np.setdiff1d(rows, init)
    Kd[:, torch.from_numpy(rows).to(Kd.device)] = 0
    _, a, _, _ = gpu_cluster(Kd, 16, C, 1)
    a = a.cpu().numpy()
    assert np.all(a[:, rows] == 0)
    Kf = Kd.float().cpu().numpy().astype(np.float64)
    mode = oracle.MIRROR if dtype == "bf16" else oracle.EXACT
    for h in range(H):
        a_o, m_o = oracle.assign(Kf[h], 16, oracle.init_centroids(Kf[h], 16, C), mode=mode)
        assert np.all(a_o[rows] == 0) and np.all(m_o[rows] == 0.0)
