"""GPU: selection quality of the cluster-granular selection on the 32k layer.

For each query head h, with the dense attention weights p_h = softmax(q_h K^T
/ sqrt(d)) over all L tokens (the problem formulation's ideal I_T keeps the
B tokens of largest q.k), two quantities of the GPU's selection S (the rows
idx[g][:n_sel[g]] of the head's KV group):
  * attention mass captured, sum_{t in S} p_h(t) (1 minus the error bound of
    the sparse output);
  * recall of the ideal set, |S cap I_T| / B, I_T the B largest q_h . k_t.
Both are reported beside a uniformly random choice of B tokens, and must
rise with the budget. The exact scores are numpy fp64 on the host.
"""
import numpy as np
import pytest
import torch

import sparse_decode_attention_ckv_amd as ck
import synth
from tests.gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu


def selection_quality(qf, Kf, idx, n_sel, G, B, rng):
    """Mean attention mass and recall of the selected rows over the query
    heads; the same for a random choice of B rows."""
    H, L, d = Kf.shape
    mass, rec, mass_r, rec_r = [], [], [], []
    for h in range(H):
        sel = idx[h, :n_sel[h]]
        rnd = rng.choice(L, size=min(B, L), replace=False)
        for g in range(G):
            z = Kf[h] @ qf[h * G + g] / np.sqrt(d)
            p = np.exp(z - z.max())
            p /= p.sum()
            top = np.argpartition(-z, B - 1)[:B]
            mass.append(p[np.unique(sel)].sum())
            rec.append(np.isin(top, sel).mean())
            mass_r.append(p[rnd].sum())
            rec_r.append(np.isin(top, rnd).mean())
    return np.mean(mass), np.mean(rec), np.mean(mass_r), np.mean(rec_r)


def test_selection_quality_rises_with_budget():
    wl = synth.workload("llama8b_layer_32k")
    say("selection quality on the 32k layer, B = 256 .. 2048")
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
        m, r, mr, rr = np.mean(acc, axis=0)
        rows.append((B, m, r, mr, rr))
        say(f"  B={B:5d}: mass {m:.3f} recall {r:.3f} | random: mass {mr:.3f} recall {rr:.3f}")
    for (B, m, r, mr, rr) in rows:
        assert m > 2 * mr and r > 2 * rr, B        # far better than chance
    assert all(rows[i + 1][1] >= rows[i][1] for i in range(len(rows) - 1))
    assert all(rows[i + 1][2] >= rows[i][2] - 0.02 for i in range(len(rows) - 1))
