"""GPU parity of the cluster-granular cache of selected KV rows.

"ClusterKV: Manipulating LLM KV Cache in Semantic Space for Recallable
Compression", section 缓存选中Token的KV with Fig. 5: the KV stays in host
memory; the GPU keeps the rows selected in the last R steps and reads only
the missing ones. A decode stream (AR(1) queries, so consecutive selections
overlap) runs ckv_select, then ckv_cache_step with K/V in pinned host memory,
then ckv_sparse_attn over the cache. At every step:
  * idx_cache, the slot tokens, the statistics and the ring equal the cache
    oracle's, fed the GPU's own selection, labels and CSR (exact);
  * every cached K/V row equals the host row of its token (bitwise);
  * the attention over the cache equals the attention over the
    device-resident K/V with the selection's idx (bitwise: same rows, same
    order).
"""
import numpy as np
import pytest
import torch

from oracle import cache as oc
import sparse_decode_attention_ckv_amd as ck
import synth
from tests.gpu_helpers import DEV, say, to_dev

pytestmark = pytest.mark.gpu


def _setup(wl, L, heads, C, host=True):
    K, V, _ = synth.make_kv(wl, L=L, heads=heads)
    Kd, Vd = to_dev(K, wl.dtype), to_dev(V, wl.dtype)
    cent, asg, off, tok = ck.ckv_cluster(Kd, wl.n_sink, C, wl.iters)
    if host:
        Ks = torch.empty(Kd.shape, dtype=Kd.dtype, pin_memory=True)
        Vs = torch.empty(Vd.shape, dtype=Vd.dtype, pin_memory=True)
        Ks.copy_(Kd.cpu())
        Vs.copy_(Vd.cpu())
    else:
        Ks, Vs = Kd.clone(), Vd.clone()
    torch.cuda.synchronize()
    return Kd, Vd, Ks, Vs, cent, asg, off, tok


def _run_stream(wl, L, heads, C, B, R, steps, rho, host=True):
    Kd, Vd, Ks, Vs, cent, asg, off, tok = _setup(wl, L, heads, C, host)
    H = len(heads)
    qs, _ = synth.make_query_stream(wl, steps, rho, heads=heads)
    Q = to_dev(qs.reshape(-1, wl.d), wl.dtype).reshape(steps, H * wl.G, wl.d)
    desc = ck.cache_desc(Ks, asg, off, tok, C, B, R, n_sink=wl.n_sink)
    st = ck.cache_state(desc, DEV)
    rows = st["rows"]
    asg_n, off_n, tok_n = asg.cpu().numpy(), off.cpu().numpy(), tok.cpu().numpy()
    Kh = Ks.cpu().view(torch.int16).numpy()
    Vh = Vs.cpu().view(torch.int16).numpy()
    hist, totals = [], np.zeros(4, dtype=np.int64)
    for t in range(steps):
        idx, ns = ck.ckv_select(Q[t], cent, off, tok, C, B, n_sink=wl.n_sink)
        cK, cV = ck.ckv_cache_step(desc, t, idx, ns, asg, off, tok, Ks, Vs, st)
        o_c = ck.ckv_sparse_attn(Q[t], cK, cV, st["idx_cache"], ns, kv_rows=rows)
        o_d = ck.ckv_sparse_attn(Q[t], Kd, Vd, idx, ns)
        # the same rows read directly from pinned host memory (no cache)
        o_h = ck.ckv_sparse_attn(Q[t], Ks, Vs, idx, ns) if host else o_d
        torch.cuda.synchronize()
        assert torch.equal(o_h, o_d), t
        idx_n, ns_n = idx.cpu().numpy(), ns.cpu().numpy()
        want = oc.step(hist, idx_n, ns_n, asg_n, off_n, tok_n, wl.n_sink, R)
        hist = want["history"]
        assert np.array_equal(st["idx_cache"].cpu().numpy(), want["idx_cache"]), t
        stats = st["stats"].cpu().numpy()
        assert np.array_equal(stats[:, :4], want["stats"]), (t, stats, want["stats"])
        assert np.all(stats[:, 4] == 0), t
        ctok = st["cache_tok"][t & 1].cpu().numpy()
        cKn = cK.cpu().view(torch.int16).numpy()
        cVn = cV.cpu().view(torch.int16).numpy()
        for h in range(H):
            n = len(want["cache_tok"][h])
            assert np.array_equal(ctok[h, :n], want["cache_tok"][h]), (t, h)
            assert np.all(ctok[h, n:] == -1), (t, h)
            assert np.array_equal(cKn[h, :n], Kh[h, ctok[h, :n]]), (t, h)
            assert np.array_equal(cVn[h, :n], Vh[h, ctok[h, :n]]), (t, h)
        ring = st["ring"].cpu().numpy()
        for k, cnt in enumerate(hist):
            s = t - len(hist) + 1 + k
            assert np.array_equal(ring[:, :C, s % R], cnt), (t, s)
        assert torch.equal(o_c, o_d), t
        totals += want["stats"].sum(axis=0)
    return totals


@pytest.mark.parametrize("R", [1, 2, 3])
def test_cache_stream_small(R):
    wl = synth.workload(1)
    say(f"cache parity: 2 heads, L=2064, C=25, B=256, R={R}, 12 steps, pinned host K/V")
    tot = _run_stream(wl, 2064, [0, 1], 25, 256, R, 12, 0.8)
    say(f"  rows hit {tot[0]}, loaded {tot[1]}; clusters hit {tot[2]} of {tot[3]}")
    assert tot[0] > 0 and tot[1] > 0


def test_cache_stream_device_source_and_many_clusters():
    wl = synth.workload(1)
    say("cache parity: 3 heads, L=8208, C=600, B=512, R=2, device-memory K/V source")
    _run_stream(wl, 8208, [0, 1, 2], 600, 512, 2, 8, 0.9, host=False)


def test_cache_stream_full_size():
    wl = synth.workload("llama8b_layer_32k")
    for R in (1, 2):
        say(f"cache parity: the 32k layer, 8 heads, C=409, B=1024, R={R}, 16 steps")
        tot = _run_stream(wl, wl.L, list(range(wl.H)), wl.C, wl.B, R, 16, 0.9)
        say(f"  rows hit {tot[0]}, loaded {tot[1]} "
            f"({tot[0] / max(1, tot[0] + tot[1]):.3f} of cluster rows from the cache)")


def test_cache_in_a_graph_replays():
    """The decode loop (select, cache step, attention) captured once and
    replayed: the ring is zeroed by a fill kernel inside the graph, so every
    replay restarts the sequence and must repeat the eager results."""
    wl = synth.workload(1)
    heads, C, B, R, steps = [0, 1], 25, 256, 2, 6
    say("cache in a graph: 2 heads, R=2, 6 steps, 3 replays")
    Kd, Vd, Ks, Vs, cent, asg, off, tok = _setup(wl, 2064, heads, C)
    qs, _ = synth.make_query_stream(wl, steps, 0.8, heads=heads)
    Q = to_dev(qs.reshape(-1, wl.d), wl.dtype).reshape(steps, len(heads) * wl.G, wl.d)
    desc = ck.cache_desc(Ks, asg, off, tok, C, B, R, n_sink=wl.n_sink)
    st = ck.cache_state(desc, DEV)
    idx = torch.empty((steps, len(heads), B), dtype=torch.int32, device=DEV)
    ns = torch.empty((steps, len(heads)), dtype=torch.int32, device=DEV)
    O = torch.empty((steps, len(heads) * wl.G, wl.d), dtype=torch.float32, device=DEV)
    ws_s = torch.empty(max(ck.ckv_select_workspace(ck.SelectDesc(
        H=len(heads), G=wl.G, d=wl.d, C=C, c_cap=C, n_sink=wl.n_sink, t_cap=tok.shape[1],
        pending_begin=0, n_pending=0, B=B, dtype=ck.CKV_BF16)), 1), dtype=torch.uint8,
        device=DEV)
    ws_a = torch.empty(ck.ckv_attn_workspace(ck.AttnDesc(
        H=len(heads), G=wl.G, d=wl.d, B=B, kv_head_stride=st["rows"] * wl.d,
        kv_rows=st["rows"], scale=0.0, dtype=ck.CKV_BF16)), dtype=torch.uint8, device=DEV)

    def loop():
        st["ring"].zero_()
        for t in range(steps):
            ck.ckv_select(Q[t], cent, off, tok, C, B, n_sink=wl.n_sink, idx=idx[t], n_sel=ns[t],
                          workspace=ws_s)
            cK, cV = ck.ckv_cache_step(desc, t, idx[t], ns[t], asg, off, tok, Ks, Vs, st)
            ck.ckv_sparse_attn(Q[t], cK, cV, st["idx_cache"], ns[t], kv_rows=st["rows"],
                               out=O[t], workspace=ws_a)

    loop()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (idx, ns, O, st["cache_K"], st["cache_V"], st["cache_tok"],
                               st["ring"])]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        got = (idx, ns, O, st["cache_K"], st["cache_V"], st["cache_tok"], st["ring"])
        for a, b in zip(ref, got):
            assert torch.equal(a, b), rep
        torch.ones(256, device=DEV).cumsum(0)         # eager work between replays
        torch.cuda.synchronize()


def test_cache_fp32_single_head():
    """The fp32 path (512-byte rows) on the single-head fp32 workload."""
    wl = synth.workload(0)
    say("cache parity: single-head fp32 2k, C=25, B=256, R=2, 10 steps, pinned host K/V")
    tot = _run_stream(wl, wl.L, [0], wl.C, wl.B, 2, 10, 0.8)
    assert tot[0] > 0 and tot[1] > 0


def test_pageable_host_memory_is_refused():
    """K/V in ordinary (pageable) host memory has no device mapping: the
    library refuses it before anything is enqueued."""
    wl = synth.workload(1)
    say("cache: pageable host K/V refused")
    K, V, _ = synth.make_kv(wl, L=200, heads=[0])
    Kd = to_dev(K, wl.dtype)
    cent, asg, off, tok = ck.ckv_cluster(Kd, wl.n_sink, 2, 2)
    Kp, Vp = Kd.cpu(), to_dev(V, wl.dtype).cpu()          # not pinned
    assert not Kp.is_pinned()
    desc = ck.cache_desc(Kp, asg, off, tok, 2, 64, 1, n_sink=wl.n_sink)
    st = ck.cache_state(desc, DEV)
    idx, ns = ck.ckv_select(to_dev(synth.make_queries(wl, 0, heads=[0])[0], wl.dtype), cent, off,
                            tok, 2, 64, n_sink=wl.n_sink)
    with pytest.raises(ck.CKVError) as e:
        ck.ckv_cache_step(desc, 0, idx, ns, asg, off, tok, Kp, Vp, st)
    assert e.value.status == ck.CKV_ERR_INVALID_ARG
    with pytest.raises(ck.CKVError):
        ck.ckv_device_view(Kp)
    torch.cuda.synchronize()


@pytest.mark.parametrize("seed", range(12))
def test_cache_random_shapes(seed):
    """Seeded random heads, window, cluster count, budget, R and query
    correlation; every step checked against the oracle as above."""
    r = np.random.default_rng(7500 + seed)
    wl = synth.workload(1)
    H = int(r.integers(1, 6))
    C = int(r.integers(2, 300))
    L = wl.n_sink + int(r.integers(C, 5000))
    B = int(r.integers(wl.n_sink + 1, min(4096, L + 200)))
    R = int(r.integers(1, 9))
    steps = int(r.integers(R + 1, 14))
    rho = float(r.choice([0.0, 0.6, 0.95]))
    host = bool(seed % 4 != 3)
    say(f"cache random seed {seed}: H={H} L={L} C={C} B={B} R={R} steps={steps} rho={rho} "
        f"host={host}")
    _run_stream(wl, L, list(range(H)), C, B, R, steps, rho, host=host)
