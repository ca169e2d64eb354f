"""GPU parity at the full sizes of the batched, 128k and incremental
workloads, in the launch configurations the benchmark uses.

At these sizes the oracle checks what it can compute quickly: the last Lloyd
iteration's labels on a token sample (both sides starting from the GPU's
previous-iteration centroids, tokens under the ASSIGN_MARGIN top-2 margin excluded),
the CSR of every head bit-exact, the centroids of the GPU's partition within
1e-4, selection bit-exact for every head and step checked, and attention
within 2e-3 of the exact fp64 attention over the same rows.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_decode_attention_ckv_amd as ck
import synth
from tests.gpu_helpers import ASSIGN_MARGIN, DEV, gpu_cluster, host_f64, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

MARGIN = ASSIGN_MARGIN


def _last_iteration_parity(Kd, heads, n_sink, C, iters, check_heads, n_sample, seed):
    """GPU: iters-1 and iters iterations (one batched launch each). Returns
    the iters-iteration results after checking them."""
    H, L, _ = Kd.shape
    c_a, _, _, _ = gpu_cluster(Kd, n_sink, C, iters - 1)
    c_b, a_b, off_b, tok_b = gpu_cluster(Kd, n_sink, C, iters)
    mu_a, mu_b = host_f64(c_a), host_f64(c_b)
    a_n, off_n, tok_n = a_b.cpu().numpy(), off_b.cpu().numpy(), tok_b.cpu().numpy()
    assert np.all(a_n[:, :n_sink] == -1)
    for h in range(H):
        o_off, o_tok = oracle.csr(a_n[h], n_sink, C)
        assert np.array_equal(off_n[h], o_off), h
        assert np.array_equal(tok_n[h], o_tok), h
    sample = np.sort(np.random.default_rng(seed).choice(np.arange(n_sink, L), n_sample,
                                                        replace=False))
    excluded = 0
    for h in check_heads:
        Kf = heads[h].Kf.astype(np.float64)
        a_o, m_o = oracle.assign(Kf[sample], 0, mu_a[h], mode=oracle.MIRROR)
        keep = m_o >= MARGIN
        excluded += int((~keep).sum())
        bad = np.nonzero(keep & (a_n[h, sample] != a_o))[0]
        assert bad.size == 0, (h, sample[bad[:5]])
        mu_o = oracle.update(Kf, n_sink, a_n[h], mu_a[h], mode=oracle.MIRROR)
        assert np.abs(mu_b[h] - mu_o).max() <= 1e-4, h
    say(f"  sampled tokens excluded by the margin rule: {excluded}/"
        f"{len(check_heads) * n_sample}")
    c_c, a_c, off_c, tok_c = gpu_cluster(Kd, n_sink, C, iters)     # deterministic
    assert torch.equal(c_b, c_c) and torch.equal(a_b, a_c)
    assert torch.equal(off_b, off_c) and torch.equal(tok_b, tok_c)
    return c_b, a_b, off_b, tok_b


def _decode_parity(wl, Kd, Vd, heads, cent, off, tok, steps):
    mu, off_n, tok_n = host_f64(cent), off.cpu().numpy(), tok.cpu().numpy()
    G = wl.G
    for step in steps:
        qs, qf = synth.make_queries(wl, step)
        qd, qf = to_dev(qs, wl.dtype), qf.astype(np.float64)
        idx, ns = ck.ckv_select(qd, cent, off, tok, wl.C, wl.B)
        o = ck.ckv_sparse_attn(qd, Kd, Vd, idx, ns)
        torch.cuda.synchronize()
        o_idx, o_ns, _ = oracle.select(qf, mu, off_n, tok_n, wl.C, wl.n_sink, wl.B, G=G)
        assert np.array_equal(ns.cpu().numpy(), o_ns), step
        assert np.array_equal(idx.cpu().numpy(), o_idx), step
        o_h = host_f64(o)
        err = 0.0
        for h in range(wl.H):
            ref = oracle.attn(qf[h * G:(h + 1) * G], heads[h].Kf[None].astype(np.float64),
                              heads[h].Vf[None].astype(np.float64), o_idx[h:h + 1],
                              o_ns[h:h + 1], G=G)
            err = max(err, rel_err(o_h[h * G:(h + 1) * G], ref))
        say(f"  step {step}: attention rel err {err:.2e}")
        assert err <= 2e-3, step


def test_batch8_full_size():
    """8 sequences x 8 KV heads (64 head problems) of 32768 tokens clustered
    in one launch (C=409, 10 iterations); decode with B=2048."""
    wl = synth.workload("llama8b_layer_32k_batch8")
    say("batched layer: 64 x 32768, C=409, 10 iterations, B=2048")
    K, V, heads = synth.make_kv(wl)
    Kd, Vd = to_dev(K, wl.dtype), to_dev(V, wl.dtype)
    del K, V
    check = list(range(0, wl.H, 9))                       # 8 heads spread over the batch
    cent, _, off, tok = _last_iteration_parity(Kd, heads, wl.n_sink, wl.C, wl.iters, check,
                                               1500, 21)
    _decode_parity(wl, Kd, Vd, heads, cent, off, tok, steps=(0, wl.steps - 1))


def test_128k_full_size():
    """One layer at 131072 tokens: C=1638 clusters, 10 iterations; decode with
    B=2048 (the selection's cut among 1638 clusters)."""
    wl = synth.workload("llama8b_layer_128k")
    say("128k layer: 8 x 131072, C=1638, 10 iterations, B=2048")
    K, V, heads = synth.make_kv(wl)
    Kd, Vd = to_dev(K, wl.dtype), to_dev(V, wl.dtype)
    del K, V
    cent, _, off, tok = _last_iteration_parity(Kd, heads, wl.n_sink, wl.C, wl.iters,
                                               list(range(wl.H)), 1200, 22)
    _decode_parity(wl, Kd, Vd, heads, cent, off, tok, steps=(0, 1, wl.steps - 1))


def test_incremental_decode_full_size():
    """The 32k layer decoding 1024 steps, one new K/V row per head per step.
    Unclustered rows are pending (always selected, counted in B); after steps
    320, 640 and 960 the newest 320 rows are clustered into 4 clusters
    (10 iterations) appended to the centroids and the CSR. Selection is
    checked at every step, attention at steps around each increment."""
    wl = synth.workload("llama8b_layer_32k_incremental")
    H, G, L0, T, m, cp, it = wl.H, wl.G, wl.L, wl.append_steps, wl.m_every, wl.c_plus, wl.iters
    say(f"incremental decode: 8 x {L0} + {T} steps, increments of {m} rows -> {cp} clusters")
    Lcap = L0 + T
    K, V, heads = synth.make_kv(wl, L=L0, L_cap=Lcap)
    app = [synth.make_appended(wl, h, T) for h in range(H)]
    Kf = np.stack([np.concatenate([heads[h].Kf, app[h][2]]) for h in range(H)]).astype(np.float64)
    Vf = np.stack([np.concatenate([heads[h].Vf, app[h][3]]) for h in range(H)]).astype(np.float64)
    Kd, Vd = to_dev(K, wl.dtype), to_dev(V, wl.dtype)        # rows >= L0 are zero
    Ka = to_dev(np.stack([a[0] for a in app]), wl.dtype)     # [H][T][d] rows to append
    Va = to_dev(np.stack([a[1] for a in app]), wl.dtype)
    n_ev = T // m
    c_cap, t_cap = wl.C + cp * n_ev, (L0 - wl.n_sink) + m * n_ev
    cent = torch.zeros((H, c_cap, 128), dtype=torch.float32, device=DEV)
    off = torch.zeros((H, c_cap + 1), dtype=torch.int32, device=DEV)
    tok = torch.zeros((H, t_cap), dtype=torch.int32, device=DEV)
    asg = torch.empty((H, L0), dtype=torch.int32, device=DEV)
    ck.ckv_cluster(Kd[:, :L0], wl.n_sink, wl.C, it, centroids=cent, assign=asg,
                   csr_offsets=off, csr_tokens=tok)
    torch.cuda.synchronize()
    C, events = wl.C, 0
    host = (host_f64(cent), off.cpu().numpy(), tok.cpu().numpy())
    attn_steps = {1, 2, m, m + 1, 2 * m + 1, 3 * m, 3 * m + 1, T}
    for s in range(1, T + 1):
        Kd[:, L0 + s - 1] = Ka[:, s - 1]
        Vd[:, L0 + s - 1] = Va[:, s - 1]
        pb, npend = L0 + m * events, s - m * events
        qs, qf = synth.make_queries(wl, s - 1)
        qd, qf = to_dev(qs, wl.dtype), qf.astype(np.float64)
        idx, ns = ck.ckv_select(qd, cent, off, tok, C, wl.B, n_sink=wl.n_sink,
                                pending_begin=pb, n_pending=npend)
        o = ck.ckv_sparse_attn(qd, Kd, Vd, idx, ns)
        torch.cuda.synchronize()
        o_idx, o_ns, _ = oracle.select(qf, host[0], host[1], host[2], C, wl.n_sink, wl.B, G=G,
                                       pending_begin=pb, n_pending=npend)
        assert np.array_equal(ns.cpu().numpy(), o_ns), s
        assert np.array_equal(idx.cpu().numpy(), o_idx), s
        if s in attn_steps:
            err = rel_err(host_f64(o), oracle.attn(qf, Kf, Vf, o_idx, o_ns, G=G))
            say(f"  step {s}: C={C}, pending {npend}, attention rel err {err:.2e}")
            assert err <= 2e-3, s
        if s % m == 0:
            base = L0 + s - m
            win = Kd[:, base:base + m]
            # iteration it-1 of the same increment, in scratch buffers
            c9, _, _, _ = gpu_cluster(win, 0, cp, it - 1, token_base=base)
            mu9 = host_f64(c9)
            a_w = torch.empty((H, m), dtype=torch.int32, device=DEV)
            ck.ckv_cluster(win, 0, cp, it, token_base=base, centroids=cent, assign=a_w,
                           csr_offsets=off, csr_tokens=tok, c_base=C, t_base=base - wl.n_sink)
            torch.cuda.synchronize()
            a_n = a_w.cpu().numpy()
            new = (host_f64(cent), off.cpu().numpy(), tok.cpu().numpy())
            assert np.array_equal(new[0][:, :C], host[0][:, :C])          # earlier state kept
            assert np.array_equal(new[1][:, :C + 1], host[1][:, :C + 1])
            assert np.array_equal(new[2][:, :base - wl.n_sink], host[2][:, :base - wl.n_sink])
            ex = 0
            for h in range(H):
                Kw = Kf[h, base:base + m]
                a_o, m_o = oracle.assign(Kw, 0, mu9[h], mode=oracle.MIRROR)
                keep = m_o >= MARGIN
                ex += int((~keep).sum())
                assert np.array_equal(a_n[h][keep], a_o[keep]), (s, h)
                o_off, o_tok = oracle.csr(a_n[h], 0, cp, token_base=base)
                assert np.array_equal(new[1][h, C:C + cp + 1], o_off + (base - wl.n_sink)), (s, h)
                assert np.array_equal(new[2][h, base - wl.n_sink:base - wl.n_sink + m], o_tok)
                mu_o = oracle.update(Kw, 0, a_n[h], mu9[h], mode=oracle.MIRROR)
                assert np.abs(new[0][h, C:C + cp] - mu_o).max() <= 1e-4, (s, h)
            say(f"  increment after step {s}: window {base}..{base + m - 1}, "
                f"excluded by the margin rule {ex}/{H * m}")
            C += cp
            events += 1
            host = new
    assert C == c_cap and events == n_ev
