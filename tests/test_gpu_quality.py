"""GPU: selection quality of the cluster-granular selection on the 32k layer.

For each query head h, with the dense attention weights p_h = softmax(q_h K^T
/ sqrt(d)) over all L tokens (the problem formulation's ideal I_T keeps the
B tokens of largest q.k), two quantities of the GPU's selection S (the rows
idx[g][:n_sel[g]] of the head's KV group):
  * attention mass captured, sum_{t in S} p_h(t) (1 minus the error bound of
    the sparse output);
  * recall of the ideal set, |S cap I_T| / B, I_T the B largest q_h . k_t.
Both are reported beside a uniformly random choice of B tokens and beside a
page-granular choice, and must rise with the budget. The page comparator
follows the page-level recall that "ClusterKV: Manipulating LLM KV Cache in
Semantic Space for Recallable Compression" argues against (section
背景知识与设计原则, Fig. 3b): the non-sink tokens in fixed pages of 16
consecutive positions, each page scored from the per-channel extremes of its
keys (channel j contributes max(q_j max_t k_tj, q_j min_t k_tj), an upper bound
of q.k over the page), the sinks plus the best pages until the budget. It
scores with the same summed query of the KV group as the cluster selection.
The exact scores are numpy fp64 on the host.
"""
import dataclasses

import numpy as np
import pytest
import torch

import sparse_decode_attention_ckv_amd as ck
import synth
from tests.gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu


def page_select(qg, Kh, n_sink, B, page=16):
    """Sinks plus the pages of largest per-channel upper bound until B rows."""
    L, d = Kh.shape
    npg = (L - n_sink) // page
    Kp = Kh[n_sink:n_sink + npg * page].reshape(npg, page, d)
    bound = np.maximum(qg * Kp.max(axis=1), qg * Kp.min(axis=1)).sum(axis=1)
    take = max(0, (B - n_sink) // page)
    best = np.argsort(-bound, kind="stable")[:take]
    rows = (n_sink + best[:, None] * page + np.arange(page)[None, :]).ravel()
    return np.concatenate([np.arange(n_sink), rows])


def selection_quality(qf, Kf, idx, n_sel, G, B, rng, n_sink=16):
    """Mean attention mass and recall of the selected rows over the query
    heads; the same for a random choice of B rows."""
    H, L, d = Kf.shape
    mass, rec, mass_r, rec_r, mass_p, rec_p = [], [], [], [], [], []
    for h in range(H):
        sel = idx[h, :n_sel[h]]
        rnd = rng.choice(L, size=min(B, L), replace=False)
        pgs = page_select(qf[h * G:(h + 1) * G].sum(axis=0), Kf[h], n_sink, B)
        for g in range(G):
            z = Kf[h] @ qf[h * G + g] / np.sqrt(d)
            p = np.exp(z - z.max())
            p /= p.sum()
            top = np.argpartition(-z, B - 1)[:B]
            mass.append(p[np.unique(sel)].sum())
            rec.append(np.isin(top, sel).mean())
            mass_r.append(p[rnd].sum())
            rec_r.append(np.isin(top, rnd).mean())
            mass_p.append(p[pgs].sum())
            rec_p.append(np.isin(top, pgs).mean())
    return (np.mean(mass), np.mean(rec), np.mean(mass_r), np.mean(rec_r), np.mean(mass_p),
            np.mean(rec_p))


@pytest.mark.parametrize("outliers", [True, False])
def test_selection_quality_rises_with_budget(outliers):
    wl = synth.workload("llama8b_layer_32k")
    if not outliers:
        wl = dataclasses.replace(wl, n_outliers=0)
    say(f"selection quality on the 32k layer ({'with' if outliers else 'without'} outlier "
        "channels), B = 256 .. 2048")
    K, V, hs = synth.make_kv(wl)
    Kd = to_dev(K, "bf16")
    Kf = np.stack([h.Kf for h in hs]).astype(np.float64)
    cent, _, off, tok = ck.ckv_cluster(Kd, 16, wl.C, wl.iters)
    rng = np.random.default_rng(3)
    rows = []
    for B in (256, 512, 1024, 2048):
        acc = []
        for step in range(3):
            qs, qf = synth.make_queries(wl, step)
            idx, ns = ck.ckv_select(to_dev(qs, "bf16"), cent, off, tok, wl.C, B)
            torch.cuda.synchronize()
            acc.append(selection_quality(qf.astype(np.float64), Kf, idx.cpu().numpy(),
                                         ns.cpu().numpy(), wl.G, B, rng))
        m, r, mr, rr, mp, rp = np.mean(acc, axis=0)
        rows.append((B, m, r, mr, rr, mp, rp))
        say(f"  B={B:5d}: mass {m:.3f} recall {r:.3f} | random: mass {mr:.3f} recall {rr:.3f} "
            f"| pages of 16: mass {mp:.3f} recall {rp:.3f}")
    for (B, m, r, mr, rr, mp, rp) in rows:
        # the ideal set: recalled far above chance and above page-granular recall
        assert r > 2 * rr and r > rp, B
        assert m > mr, B
        if outliers:
            assert m > 2 * mr, B
    assert all(rows[i + 1][1] >= rows[i][1] for i in range(len(rows) - 1))
    if outliers:
        assert all(rows[i + 1][2] >= rows[i][2] - 0.02 for i in range(len(rows) - 1))
