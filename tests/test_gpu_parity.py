"""GPU parity: every call of the C ABI against the CPU oracle on the same
seeded inputs (tolerances: selection and CSR bit-exact; per-iteration Lloyd
labels bit-exact outside the ASSIGN_MARGIN top-2 margin; centroids max abs 1e-4;
attention max relative error 2e-3 for bf16 and 1e-5 for fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_decode_attention_ckv_amd as ck
import synth
from tests.gpu_helpers import (ASSIGN_MARGIN, DEV, gpu_cluster, host_f64, lloyd_parity, rel_err, say,
                               to_dev)

pytestmark = pytest.mark.gpu

D = 128


def _kv(wl, L, heads=None):
    K, V, hs = synth.make_kv(wl, L=L, heads=heads)
    Kf = np.stack([h.Kf for h in hs]).astype(np.float64)
    Vf = np.stack([h.Vf for h in hs]).astype(np.float64)
    return to_dev(K, wl.dtype), to_dev(V, wl.dtype), Kf, Vf


def _q(wl, step, heads=None):
    qs, qf = synth.make_queries(wl, step, heads=heads)
    return to_dev(qs, wl.dtype), qf.astype(np.float64)


def _random_idx(rng, H, B, L, n_sink, n_sel):
    idx = np.full((H, B), -1, np.int32)
    for h in range(H):
        n = n_sel[h]
        rest = rng.choice(np.arange(n_sink, L), size=max(n - n_sink, 0), replace=False)
        row = np.concatenate([np.arange(min(n_sink, n)), rest])[:n]
        idx[h, :n] = row
    return idx


# ------------------------------------------------------------- attention --

@pytest.mark.parametrize("wl_id,H,G,L,B,tol", [
    (0, 1, 1, 2048, 256, 1e-5),      # single-head fp32 workload shape
    (1, 2, 4, 3000, 1000, 2e-3),     # bf16, GQA 4, ragged B
    (1, 3, 1, 700, 64, 2e-3),
])
def test_attention_parity(wl_id, H, G, L, B, tol):
    wl = synth.workload(wl_id)
    say(f"attention parity wl={wl.name} H={H} G={G} L={L} B={B}")
    Kd, Vd, Kf, Vf = _kv(wl, L, heads=range(H))
    rng = np.random.default_rng(1)
    qs = rng.standard_normal((H * G, D)) * 3
    qs[:, 7] *= 20
    if wl.dtype == "bf16":
        qbits = synth.bf16_bits(qs)
        qd, qf = to_dev(qbits, "bf16"), synth.bf16_to_f32(qbits).astype(np.float64)
    else:
        qd, qf = to_dev(qs.astype(np.float32), "f32"), qs.astype(np.float32).astype(np.float64)
    n_sel = np.array([B - (37 * h) % B for h in range(H)], np.int32)   # ragged per head
    idx = _random_idx(rng, H, B, L, 16, n_sel)
    o = ck.ckv_sparse_attn(qd, Kd, Vd, torch.from_numpy(idx).to(DEV),
                           torch.from_numpy(n_sel).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.attn(qf, Kf, Vf, idx, n_sel, G=G)
    err = rel_err(host_f64(o), ref)
    say(f"  rel err {err:.3e}")
    assert err <= tol


def test_attention_all_rows_equals_dense():
    wl = synth.workload(0)
    say("attention: every row selected equals dense attention (fp32)")
    Kd, Vd, Kf, Vf = _kv(wl, 2048)
    qd, qf = _q(wl, 0)
    L = 2048
    idx = np.random.default_rng(2).permutation(L).astype(np.int32)[None]
    o = ck.ckv_sparse_attn(qd, Kd, Vd, torch.from_numpy(idx).to(DEV),
                           torch.tensor([L], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    ref = oracle.dense_attn(qf, Kf, Vf)
    assert rel_err(host_f64(o), ref) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_edge_cases(dtype):
    say(f"attention edge cases {dtype}")
    wl = synth.workload(0 if dtype == "f32" else 1)
    H, G, L, B = 4, 2, 200, 70
    Kd, Vd, Kf, Vf = _kv(wl, L, heads=range(H))
    rng = np.random.default_rng(3)
    qs = rng.standard_normal((H * G, D))
    qd = to_dev(synth.bf16_bits(qs) if dtype == "bf16" else qs.astype(np.float32), dtype)
    idx = np.full((H, B), -1, np.int32)
    idx[1, 0] = 17                       # one row -> exactly its value
    idx[2, :5] = [3, 9, 250, -7, 11]     # out-of-range entries are skipped
    idx[3, :B] = rng.integers(0, L, B)   # full budget, repeats allowed
    n_sel = np.array([0, 1, 5, B], np.int32)
    o = ck.ckv_sparse_attn(qd, Kd, Vd, torch.from_numpy(idx).to(DEV),
                           torch.from_numpy(n_sel).to(DEV), kv_rows=L)
    torch.cuda.synchronize()
    o = host_f64(o)
    assert np.all(o[0:G] == 0.0)
    assert np.array_equal(o[G:2 * G], np.tile(Vf[1, 17], (G, 1)))
    qf = host_f64(qd)
    kept = np.array([[3, 9, 11]], np.int32)
    ref2 = oracle.attn(qf[2 * G:3 * G], Kf[2:3], Vf[2:3], kept, [3], G=G)
    assert rel_err(o[2 * G:3 * G], ref2) <= (1e-5 if dtype == "f32" else 2e-3)
    ref3 = oracle.attn(qf[3 * G:], Kf[3:4], Vf[3:4], idx[3:4], [B], G=G)
    assert rel_err(o[3 * G:], ref3) <= (1e-5 if dtype == "f32" else 2e-3)


# -------------------------------------------------------------- selection --

def _random_csr(rng, H, C, Lp, n_sink, c_cap=None, t_cap=None):
    c_cap = C if c_cap is None else c_cap
    t_cap = Lp if t_cap is None else t_cap
    off = np.zeros((H, c_cap + 1), np.int32)
    tok = np.zeros((H, t_cap), np.int32)
    for h in range(H):
        a = rng.integers(0, C, size=n_sink + Lp).astype(np.int32)
        a[:n_sink] = -1
        o, t = oracle.csr(a, n_sink, C)
        off[h, :C + 1] = o
        off[h, C + 1:] = o[-1]
        tok[h, :Lp] = t
    return off, tok


@pytest.mark.parametrize("H,G,C,Lp,B,n_sink,n_pending,dtype", [
    (8, 4, 409, 32752, 1024, 16, 0, "bf16"),     # llama8b 32k layer shape
    (2, 1, 25, 2032, 256, 16, 0, "f32"),         # single-head fp32 shape
    (3, 4, 1638, 20000, 2048, 16, 0, "bf16"),    # 2048-wide sort
    (2, 4, 2048, 4096, 300, 16, 0, "bf16"),      # maximum C
    (2, 4, 1, 500, 100, 16, 0, "bf16"),          # single cluster
    (2, 4, 57, 900, 16, 16, 0, "bf16"),          # B = n_sink
    (2, 4, 57, 900, 5000, 16, 0, "bf16"),        # B >= L
    (4, 4, 421, 32752, 1024, 16, 64, "bf16"),    # pending decode tokens
    (2, 8, 130, 3000, 777, 0, 0, "f32"),
])
def test_select_parity(H, G, C, Lp, B, n_sink, n_pending, dtype):
    say(f"select parity H={H} G={G} C={C} Lp={Lp} B={B} sink={n_sink} pend={n_pending} {dtype}")
    rng = np.random.default_rng(C + B)
    mu = (rng.standard_normal((H, C, D)) * 2).astype(np.float32)
    mu[:, :, 7] *= 20
    off, tok = _random_csr(rng, H, C, Lp, n_sink)
    qs = rng.standard_normal((H * G, D)) * 3
    if dtype == "bf16":
        qb = synth.bf16_bits(qs)
        qd, qf = to_dev(qb, "bf16"), synth.bf16_to_f32(qb).astype(np.float64)
    else:
        qd, qf = to_dev(qs.astype(np.float32), "f32"), qs.astype(np.float32).astype(np.float64)
    pb = n_sink + Lp
    idx, ns = ck.ckv_select(qd, torch.from_numpy(mu).to(DEV), torch.from_numpy(off).to(DEV),
                            torch.from_numpy(tok).to(DEV), C, B, n_sink=n_sink,
                            pending_begin=pb, n_pending=n_pending)
    torch.cuda.synchronize()
    o_idx, o_ns, _ = oracle.select(qf, mu.astype(np.float64), off, tok, C, n_sink, B, G=G,
                                   pending_begin=pb, n_pending=n_pending)
    assert np.array_equal(ns.cpu().numpy(), o_ns)
    assert np.array_equal(idx.cpu().numpy(), o_idx)


def test_select_exact_ties_go_to_lower_id():
    say("select: equal scores rank by lower cluster id")
    rng = np.random.default_rng(5)
    H, G, C, Lp = 2, 4, 40, 400
    base = rng.standard_normal((5, D)).astype(np.float32)
    mu = base[rng.integers(0, 5, size=(H, C))]          # many exact duplicates
    off, tok = _random_csr(rng, H, C, Lp, 16)
    qb = synth.bf16_bits(rng.standard_normal((H * G, D)))
    qd, qf = to_dev(qb, "bf16"), synth.bf16_to_f32(qb).astype(np.float64)
    for B in (16, 40, 131, 416):
        idx, ns = ck.ckv_select(qd, torch.from_numpy(mu).to(DEV), torch.from_numpy(off).to(DEV),
                                torch.from_numpy(tok).to(DEV), C, B)
        torch.cuda.synchronize()
        o_idx, o_ns, _ = oracle.select(qf, mu.astype(np.float64), off, tok, C, 16, B, G=G)
        assert np.array_equal(idx.cpu().numpy(), o_idx), B
    # q = 0: every score is exactly zero, the cluster id alone decides
    qz = torch.zeros_like(qd)
    for B in (17, 200, 416):
        idx, ns = ck.ckv_select(qz, torch.from_numpy(mu).to(DEV), torch.from_numpy(off).to(DEV),
                                torch.from_numpy(tok).to(DEV), C, B)
        torch.cuda.synchronize()
        o_idx, o_ns, _ = oracle.select(np.zeros_like(qf), mu.astype(np.float64), off, tok, C, 16,
                                       B, G=G)
        assert np.array_equal(idx.cpu().numpy(), o_idx), ("q=0", B)


def test_select_crowded_score_bucket():
    """One cluster's score dwarfs the rest, so the others crowd into a few of
    the equal-width score buckets and the cut is found by the exact passes
    over the rank key; also near-equal scores (relative spread about 1e-6)."""
    say("select: crowded score buckets (outlier cluster, near-equal scores)")
    rng = np.random.default_rng(17)
    H, G, C, Lp = 3, 4, 300, 6000
    off, tok = _random_csr(rng, H, C, Lp, 16)
    qb = synth.bf16_bits(rng.standard_normal((H * G, D)))
    qd, qf = to_dev(qb, "bf16"), synth.bf16_to_f32(qb).astype(np.float64)
    mu_out = rng.standard_normal((H, C, D)).astype(np.float32)
    for h in range(H):
        mu_out[h, 5 + h] *= 3e6 * (1 if h != 1 else -1)    # top outlier, or bottom for h = 1
    base = rng.standard_normal((H, 1, D))
    mu_near = (base * (1 + 1e-6 * rng.standard_normal((H, C, D)))).astype(np.float32)
    for mu in (mu_out, mu_near):
        for B in (40, 333, 1500):
            idx, ns = ck.ckv_select(qd, torch.from_numpy(mu).to(DEV),
                                    torch.from_numpy(off).to(DEV), torch.from_numpy(tok).to(DEV),
                                    C, B)
            torch.cuda.synchronize()
            o_idx, o_ns, _ = oracle.select(qf, mu.astype(np.float64), off, tok, C, 16, B, G=G)
            assert np.array_equal(ns.cpu().numpy(), o_ns), B
            assert np.array_equal(idx.cpu().numpy(), o_idx), B


# ------------------------------------------------------------- clustering --

def test_cluster_fp32_single_head_per_iteration():
    wl = synth.workload(0)
    say("cluster parity: single-head fp32 2k, 10 iterations (EXACT oracle)")
    Kd, _, Kf, _ = _kv(wl, wl.L)
    ex = lloyd_parity(Kd, Kf, wl.n_sink, wl.C, wl.iters, oracle.EXACT)
    say(f"  excluded (margin < {ASSIGN_MARGIN}) per iteration: {ex}")


@pytest.mark.parametrize("H,L,C", [(2, 4112, 51), (1, 1000, 7), (3, 2600, 64)])
def test_cluster_bf16_per_iteration(H, L, C):
    wl = synth.workload(1)
    say(f"cluster parity bf16 H={H} L={L} C={C} (MIRROR oracle)")
    Kd, _, Kf, _ = _kv(wl, L, heads=range(H))
    lloyd_parity(Kd, Kf, 16, C, 6, oracle.MIRROR)


def test_cluster_edge_cases():
    wl = synth.workload(1)
    say("cluster edge cases: C=1, C=L', n_sink=0, tiny windows")
    Kd, _, Kf, _ = _kv(wl, 300, heads=range(2))
    # C = 1: every non-sink key in one cluster, centroid = mean
    cent, asg, off, tok = gpu_cluster(Kd, 16, 1, 2)
    assert np.all(asg.cpu().numpy()[:, 16:] == 0)
    np.testing.assert_allclose(host_f64(cent)[:, 0], Kf[:, 16:].mean(axis=1), atol=1e-4)
    # C = L': every key its own cluster
    lloyd_parity(Kd[:, :80].contiguous(), Kf[:, :80], 16, 64, 2, oracle.MIRROR)
    # no sinks, C + increment-sized window
    lloyd_parity(Kd[:, :320].contiguous(), Kf[:, :320], 0, 4, 10, oracle.MIRROR)
    # window shorter than one tile of the assignment kernel
    lloyd_parity(Kd[:, :40].contiguous(), Kf[:, :40], 3, 5, 3, oracle.MIRROR)


def test_cluster_append_increment():
    """Decode-time increments: a 320-token window clustered into 4 clusters
    and appended after the prompt's clusters in the same CSR."""
    wl = synth.workload(3)
    say("cluster append: prompt 2064 rows, C=25, then window 320 -> 4 clusters")
    H, L0, C0 = 2, 2064, 25
    Kd, _, Kf, _ = _kv(wl, L0 + 320, heads=range(H))
    c_cap, t_cap = C0 + 4, (L0 - 16) + 320
    cent = torch.zeros((H, c_cap, D), dtype=torch.float32, device=DEV)
    off = torch.zeros((H, c_cap + 1), dtype=torch.int32, device=DEV)
    tok = torch.zeros((H, t_cap), dtype=torch.int32, device=DEV)
    asg0 = torch.empty((H, L0), dtype=torch.int32, device=DEV)
    ck.ckv_cluster(Kd[:, :L0], 16, C0, 10, centroids=cent, assign=asg0, csr_offsets=off,
                   csr_tokens=tok)
    torch.cuda.synchronize()
    before = (host_f64(cent).copy(), off.cpu().numpy().copy(), tok.cpu().numpy().copy())
    asg1 = torch.empty((H, 320), dtype=torch.int32, device=DEV)
    win = Kd[:, L0:L0 + 320]                       # strided view into the cache
    ck.ckv_cluster(win, 0, 4, 10, token_base=L0, centroids=cent, assign=asg1,
                   csr_offsets=off, csr_tokens=tok, c_base=C0, t_base=L0 - 16)
    torch.cuda.synchronize()
    mu, o, t = host_f64(cent), off.cpu().numpy(), tok.cpu().numpy()
    assert np.array_equal(mu[:, :C0], before[0][:, :C0])
    assert np.array_equal(o[:, :C0 + 1], before[1][:, :C0 + 1])
    assert np.array_equal(t[:, :L0 - 16], before[2][:, :L0 - 16])
    for h in range(H):
        r = oracle.cluster(Kf[h, L0:L0 + 320], 0, 4, 10, mode=oracle.MIRROR, token_base=L0)
        a_g = asg1.cpu().numpy()[h]
        o_off, o_tok = oracle.csr(a_g, 0, 4, token_base=L0)
        assert np.array_equal(o[h, C0:], o_off + (L0 - 16))
        assert np.array_equal(t[h, L0 - 16:], o_tok)
        say(f"  head {h}: labels equal to an independent oracle run: "
            f"{np.mean(a_g == r['assign']):.4f}")


@pytest.mark.parametrize("seed", range(8))
def test_cluster_append_random(seed):
    """Seeded appends: prompt and window lengths, cluster counts (even seeds
    through the one-launch small-window kernel, odd ones through the general
    path), window sinks, iterations, and a strided window view into the cache.
    The appended segment must be bitwise the window clustered alone, shifted
    by c_base, t_base and token_base, and nothing before it may change."""
    r = np.random.default_rng(7700 + seed)
    wl = synth.workload(3)
    H = int(r.integers(1, 4))
    L0 = int(r.integers(600, 4000))
    C0 = int(r.integers(2, 300))
    small = seed % 2 == 0
    ws = int(r.choice([0, 0, 5]))
    Lw = ws + (int(r.integers(40, 1025)) if small else int(r.integers(1100, 3000)))
    Cw = int(r.integers(1, 17)) if small else int(r.integers(17, 300))
    iters = int(r.integers(1, 6))
    say(f"cluster append seed {seed}: H={H} prompt {L0} rows C={C0}, window {Lw} rows "
        f"(sinks {ws}) C={Cw}, {iters} iterations")
    Kd, _, _, _ = _kv(wl, L0 + Lw, heads=range(H))
    c_cap, t_cap = C0 + Cw, (L0 - 16) + (Lw - ws)
    cent = torch.zeros((H, c_cap, D), dtype=torch.float32, device=DEV)
    off = torch.zeros((H, c_cap + 1), dtype=torch.int32, device=DEV)
    tok = torch.zeros((H, t_cap), dtype=torch.int32, device=DEV)
    asg0 = torch.empty((H, L0), dtype=torch.int32, device=DEV)
    ck.ckv_cluster(Kd[:, :L0], 16, C0, 3, centroids=cent, assign=asg0, csr_offsets=off,
                   csr_tokens=tok)
    torch.cuda.synchronize()
    before = (cent.clone(), off.clone(), tok.clone())
    win = Kd[:, L0:L0 + Lw]                       # strided view into the cache
    asg1 = torch.empty((H, Lw), dtype=torch.int32, device=DEV)
    ck.ckv_cluster(win, ws, Cw, iters, token_base=L0, centroids=cent, assign=asg1,
                   csr_offsets=off, csr_tokens=tok, c_base=C0, t_base=L0 - 16)
    rc, ra, ro, rt = gpu_cluster(win.contiguous(), ws, Cw, iters, token_base=L0)
    torch.cuda.synchronize()
    assert torch.equal(cent[:, :C0], before[0][:, :C0])
    assert torch.equal(off[:, :C0 + 1], before[1][:, :C0 + 1])
    assert torch.equal(tok[:, :L0 - 16], before[2][:, :L0 - 16])
    assert torch.equal(cent[:, C0:], rc)
    assert torch.equal(asg1, ra)
    assert torch.equal(off[:, C0:], ro + (L0 - 16))
    assert torch.equal(tok[:, L0 - 16:], rt)


def test_cluster_full_size_sampled_and_deterministic():
    """Llama-8B-shaped layer at 32k (8 KV heads, C=409, 10 iterations) in the
    launch configuration the benchmark times; labels checked on a token
    sample, CSR and centroids in full."""
    wl = synth.workload(1)
    say("cluster full size 8 x 32768, C=409: iterations 9 and 10")
    Kd, _, Kf, _ = _kv(wl, wl.L)
    c9, a9, _, _ = gpu_cluster(Kd, 16, wl.C, 9)
    c10, a10, off10, tok10 = gpu_cluster(Kd, 16, wl.C, 10)
    mu9, a10n = host_f64(c9), a10.cpu().numpy()
    sample = np.sort(np.random.default_rng(7).choice(np.arange(16, wl.L), 3000, replace=False))
    ex = 0
    for h in range(wl.H):
        a_o, m_o = oracle.assign(Kf[h][sample], 0, mu9[h], mode=oracle.MIRROR)
        keep = m_o >= ASSIGN_MARGIN
        ex += int((~keep).sum())
        assert np.array_equal(a10n[h, sample][keep], a_o[keep]), h
        o_off, o_tok = oracle.csr(a10n[h], 16, wl.C)
        assert np.array_equal(off10.cpu().numpy()[h], o_off)
        assert np.array_equal(tok10.cpu().numpy()[h], o_tok)
        mu_o = oracle.update(Kf[h], 16, a10n[h], mu9[h], mode=oracle.MIRROR)
        assert np.abs(host_f64(c10)[h] - mu_o).max() <= 1e-4
    say(f"  sampled tokens excluded by the margin rule: {ex}/{wl.H * len(sample)}")
    c10b, a10b, off10b, tok10b = gpu_cluster(Kd, 16, wl.C, 10)
    assert torch.equal(c10, c10b) and torch.equal(a10, a10b)
    assert torch.equal(off10, off10b) and torch.equal(tok10, tok10b)


def test_select_attention_on_gpu_clusters_full_size():
    """Decode steps of the 32k layer: selection bit-exact against the oracle
    given the GPU's centroids and CSR; attention within 2e-3 of the exact
    fp64 attention over the same rows; runs are deterministic."""
    wl = synth.workload(1)
    say("decode steps on GPU clusters, 8 x 32768, C=409, B=1024")
    Kd, Vd, Kf, Vf = _kv(wl, wl.L)
    cent, asg, off, tok = gpu_cluster(Kd, 16, wl.C, wl.iters)
    mu, offn, tokn = host_f64(cent), off.cpu().numpy(), tok.cpu().numpy()
    for step in range(4):
        qd, qf = _q(wl, step)
        idx, ns = ck.ckv_select(qd, cent, off, tok, wl.C, wl.B)
        o = ck.ckv_sparse_attn(qd, Kd, Vd, idx, ns)
        torch.cuda.synchronize()
        o_idx, o_ns, _ = oracle.select(qf, mu, offn, tokn, wl.C, 16, wl.B, G=wl.G)
        assert np.array_equal(idx.cpu().numpy(), o_idx), step
        assert np.array_equal(ns.cpu().numpy(), o_ns), step
        ref = oracle.attn(qf, Kf, Vf, o_idx, o_ns, G=wl.G)
        err = rel_err(host_f64(o), ref)
        say(f"  step {step}: rel err {err:.2e}")
        assert err <= 2e-3
        idx2, _ = ck.ckv_select(qd, cent, off, tok, wl.C, wl.B)
        o2 = ck.ckv_sparse_attn(qd, Kd, Vd, idx2, ns)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx2) and torch.equal(o, o2)


# ------------------------------------------------------------ limits --

@pytest.mark.parametrize("L,C,iters", [(6160, 2048, 2), (3016, 600, 3)])
def test_cluster_many_clusters_per_iteration(L, C, iters):
    """The largest C (2048: four 512-cluster rounds of centroids in LDS) and a
    C just past one round (600), per-iteration parity."""
    wl = synth.workload(1)
    say(f"cluster parity bf16 at many clusters: L={L} C={C}")
    Kd, _, Kf, _ = _kv(wl, L, heads=range(1))
    lloyd_parity(Kd, Kf, 16, C, iters, oracle.MIRROR)


def test_attention_largest_budget_and_strided_cache():
    """B = 32768 (512 splits, the largest supported), ragged n_sel, on K and V
    that are views into a longer cache (head stride > rows x d)."""
    wl = synth.workload(1)
    say("attention at B=32768 on strided K/V views")
    H, G, L, Lcap, B = 2, 4, 33000, 33100, 32768
    K, V, hs = synth.make_kv(wl, L=L, L_cap=Lcap, heads=range(H))
    Kd, Vd = to_dev(K, "bf16")[:, :L], to_dev(V, "bf16")[:, :L]
    assert Kd.stride(0) == Lcap * D and not Kd.is_contiguous()
    Kf = np.stack([h.Kf for h in hs]).astype(np.float64)
    Vf = np.stack([h.Vf for h in hs]).astype(np.float64)
    rng = np.random.default_rng(9)
    qb = synth.bf16_bits(rng.standard_normal((H * G, D)) * 3)
    qd, qf = to_dev(qb, "bf16"), synth.bf16_to_f32(qb).astype(np.float64)
    n_sel = np.array([B, B - 77], np.int32)
    idx = _random_idx(rng, H, B, L, 16, n_sel)
    o = ck.ckv_sparse_attn(qd, Kd, Vd, torch.from_numpy(idx).to(DEV),
                           torch.from_numpy(n_sel).to(DEV))
    torch.cuda.synchronize()
    err = rel_err(host_f64(o), oracle.attn(qf, Kf, Vf, idx, n_sel, G=G))
    say(f"  rel err {err:.2e}")
    assert err <= 2e-3


def test_single_head_fp32_end_to_end():
    """The single-head fp32 2k workload end to end on the GPU: its own
    10-iteration clustering, then selection with B = 256 on those clusters
    (bit-exact against the oracle given the GPU's centroids and CSR), then
    the sparse attention over the selected rows and the fused one-call step,
    both within 1e-5 of the fp64 oracle; with B >= L the selection takes
    every row and the output is dense decode attention, within 1e-5."""
    wl = synth.workload(0)
    say("single-head fp32 2k end to end: cluster -> select -> attention")
    Kd, Vd, Kf, Vf = _kv(wl, wl.L)
    cent, asg, off, tok = gpu_cluster(Kd, wl.n_sink, wl.C, wl.iters)
    mu, off_h, tok_h = host_f64(cent), off.cpu().numpy(), tok.cpu().numpy()
    # the CSR is the one of the GPU's labels
    o_off, o_tok = oracle.csr(asg.cpu().numpy()[0], wl.n_sink, wl.C)
    assert np.array_equal(off_h[0], o_off) and np.array_equal(tok_h[0], o_tok)
    for step in range(3):
        qd, qf = _q(wl, step)
        for B in (wl.B, wl.L, wl.L + 64):
            idx, ns = ck.ckv_select(qd, cent, off, tok, wl.C, B, n_sink=wl.n_sink)
            o = ck.ckv_sparse_attn(qd, Kd, Vd, idx, ns)
            idx2, ns2, o2 = ck.ckv_select_attn(qd, cent, off, tok, wl.C, B, Kd, Vd,
                                               n_sink=wl.n_sink)
            torch.cuda.synchronize()
            o_idx, o_ns, _ = oracle.select(qf, mu, off_h, tok_h, wl.C, wl.n_sink, B, G=wl.G)
            assert np.array_equal(idx.cpu().numpy(), o_idx), (step, B)
            assert np.array_equal(ns.cpu().numpy(), o_ns), (step, B)
            assert torch.equal(idx, idx2) and torch.equal(o, o2), (step, B)
            ref = oracle.attn(qf, Kf, Vf, o_idx, o_ns, G=wl.G)
            err = rel_err(host_f64(o), ref)
            assert err <= 1e-5, (step, B, err)
            if B >= wl.L:
                assert o_ns[0] == wl.L
                dense = oracle.dense_attn(qf, Kf, Vf, G=wl.G)
                assert rel_err(host_f64(o), dense) <= 1e-5, (step, B)
