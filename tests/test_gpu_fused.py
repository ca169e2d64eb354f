"""GPU parity of ckv_select_attn, the fused decode step: its idx, n_sel and o
must be bitwise what ckv_select followed by ckv_sparse_attn produce on the
same inputs, and match the oracle (selection bit-exact, attention within
2e-3 for bf16 and 1e-5 for fp32 of the exact fp64 attention)."""
import ctypes as ct

import numpy as np
import pytest
import torch

import oracle
import sparse_decode_attention_ckv_amd as ck
import synth
from tests.gpu_helpers import DEV, gpu_cluster, host_f64, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

D = 128


def _random_csr(rng, H, C, Lp, n_sink):
    off = np.zeros((H, C + 1), np.int32)
    tok = np.zeros((H, Lp), np.int32)
    for h in range(H):
        a = rng.integers(0, C, size=n_sink + Lp).astype(np.int32)
        a[:n_sink] = -1
        off[h], tok[h] = oracle.csr(a, n_sink, C)
    return off, tok


@pytest.mark.parametrize("H,G,C,Lp,B,n_sink,n_pending,dtype", [
    (8, 4, 409, 32752, 1024, 16, 0, "bf16"),     # llama8b 32k layer shape
    (3, 4, 1638, 20000, 2048, 16, 0, "bf16"),    # 128k-layer cluster count
    (2, 1, 57, 900, 200, 16, 0, "bf16"),         # G = 1, ragged last split
    (2, 8, 130, 3000, 777, 0, 0, "bf16"),        # G = 8, no sinks
    (4, 4, 421, 32752, 1024, 16, 64, "bf16"),    # pending decode tokens
    (2, 4, 57, 900, 5000, 16, 0, "bf16"),        # B >= L: every row selected
    (2, 4, 57, 900, 16, 16, 0, "bf16"),          # B = n_sink: sinks only
    (9, 4, 64, 1000, 130, 16, 0, "bf16"),        # H not a multiple of 8
    (64, 4, 409, 4000, 2048, 16, 0, "bf16"),     # batched grid: 2048 workgroups
    (3, 4, 1638, 8000, 3000, 16, 40, "bf16"),    # 2048-cluster LDS, pending, ragged split
    (2, 1, 25, 2032, 256, 16, 0, "f32"),         # fp32: the separate kernels
])
def test_fused_equals_separate_and_oracle(H, G, C, Lp, B, n_sink, n_pending, dtype):
    say(f"fused decode step H={H} G={G} C={C} Lp={Lp} B={B} sink={n_sink} pend={n_pending} "
        f"{dtype}")
    rng = np.random.default_rng(C * 7 + B)
    mu = (rng.standard_normal((H, C, D)) * 2).astype(np.float32)
    mu[:, :, 7] *= 20
    off, tok = _random_csr(rng, H, C, Lp, n_sink)
    L = n_sink + Lp + n_pending
    Ks = rng.standard_normal((H, L, D)) * 2
    Vs = rng.standard_normal((H, L, D))
    qs = rng.standard_normal((H * G, D)) * 3
    if dtype == "bf16":
        kb, vb, qb = synth.bf16_bits(Ks), synth.bf16_bits(Vs), synth.bf16_bits(qs)
        Kd, Vd, qd = to_dev(kb, "bf16"), to_dev(vb, "bf16"), to_dev(qb, "bf16")
        Kf, Vf, qf = (synth.bf16_to_f32(x).astype(np.float64) for x in (kb, vb, qb))
        tol = 2e-3
    else:
        k32, v32, q32 = (x.astype(np.float32) for x in (Ks, Vs, qs))
        Kd, Vd, qd = to_dev(k32, "f32"), to_dev(v32, "f32"), to_dev(q32, "f32")
        Kf, Vf, qf = (x.astype(np.float64) for x in (k32, v32, q32))
        tol = 1e-5
    mud, offd, tokd = (torch.from_numpy(x).to(DEV) for x in (mu, off, tok))
    pb = n_sink + Lp
    idx, ns = ck.ckv_select(qd, mud, offd, tokd, C, B, n_sink=n_sink, pending_begin=pb,
                            n_pending=n_pending)
    o = ck.ckv_sparse_attn(qd, Kd, Vd, idx, ns)
    fidx, fns, fo = ck.ckv_select_attn(qd, mud, offd, tokd, C, B, Kd, Vd, n_sink=n_sink,
                                       pending_begin=pb, n_pending=n_pending)
    torch.cuda.synchronize()
    assert torch.equal(fidx, idx) and torch.equal(fns, ns)
    assert torch.equal(fo, o)
    o_idx, o_ns, _ = oracle.select(qf, mu.astype(np.float64), off, tok, C, n_sink, B, G=G,
                                   pending_begin=pb, n_pending=n_pending)
    assert np.array_equal(fidx.cpu().numpy(), o_idx)
    assert np.array_equal(fns.cpu().numpy(), o_ns)
    err = rel_err(host_f64(fo), oracle.attn(qf, Kf, Vf, o_idx, o_ns, G=G))
    say(f"  rel err {err:.2e}")
    assert err <= tol


def test_fused_on_gpu_clusters_full_size_and_graph():
    """The 32k layer: the fused step on the GPU's own clusters, eager and
    replayed from a HIP graph (several replays, each checked), equal to the
    separate calls."""
    wl = synth.workload(1)
    say("fused decode step on GPU clusters, 8 x 32768, C=409, B=1024, graph replays")
    K, V, hs = synth.make_kv(wl, L=wl.L)
    Kd, Vd = to_dev(K, "bf16"), to_dev(V, "bf16")
    cent, asg, off, tok = gpu_cluster(Kd, 16, wl.C, wl.iters)
    qs, _ = synth.make_queries(wl, 0)
    qd = to_dev(qs, "bf16")
    idx, ns = ck.ckv_select(qd, cent, off, tok, wl.C, wl.B)
    o = ck.ckv_sparse_attn(qd, Kd, Vd, idx, ns)
    torch.cuda.synchronize()
    sd = ck.SelectDesc(H=wl.H, G=wl.G, d=D, C=wl.C, c_cap=wl.C, n_sink=16, t_cap=tok.shape[1],
                       pending_begin=0, n_pending=0, B=wl.B, dtype=ck.CKV_BF16)
    ad = ck.AttnDesc(H=wl.H, G=wl.G, d=D, B=wl.B, kv_head_stride=Kd.stride(0),
                     kv_rows=Kd.shape[1], scale=0.0, dtype=ck.CKV_BF16)
    ws = torch.empty(ck.ckv_select_attn_workspace(sd, ad), dtype=torch.uint8, device=DEV)
    fidx = torch.empty_like(idx)
    fns = torch.empty_like(ns)
    fo = torch.empty_like(o)

    def step():
        ck.ckv_select_attn(qd, cent, off, tok, wl.C, wl.B, Kd, Vd, idx=fidx, n_sel=fns, out=fo,
                           workspace=ws)

    step()
    torch.cuda.synchronize()
    assert torch.equal(fidx, idx) and torch.equal(fns, ns) and torch.equal(fo, o)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        fidx.fill_(-7)
        fo.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(fidx, idx) and torch.equal(fns, ns) and torch.equal(fo, o), rep


def test_host_kv_and_pageable_refusal():
    """K/V in pinned host memory: the fused step and the separate attention
    read them through their device mapping (the gather pattern for the host
    link) and give the device results bitwise. Pageable host memory is
    refused before anything is launched, by the binding and by the C entry
    points themselves."""
    say("fused and separate attention over pinned host K/V; pageable K/V refused")
    rng = np.random.default_rng(11)
    H, G, C, Lp, B, n_sink = 3, 4, 57, 3000, 700, 16
    mu = (rng.standard_normal((H, C, D)) * 2).astype(np.float32)
    off, tok = _random_csr(rng, H, C, Lp, n_sink)
    L = n_sink + Lp
    Kd = to_dev(synth.bf16_bits(rng.standard_normal((H, L, D)) * 2), "bf16")
    Vd = to_dev(synth.bf16_bits(rng.standard_normal((H, L, D))), "bf16")
    qd = to_dev(synth.bf16_bits(rng.standard_normal((H * G, D)) * 3), "bf16")
    mud, offd, tokd = (torch.from_numpy(x).to(DEV) for x in (mu, off, tok))
    Kh = torch.empty(Kd.shape, dtype=Kd.dtype, pin_memory=True)
    Vh = torch.empty(Vd.shape, dtype=Vd.dtype, pin_memory=True)
    Kh.copy_(Kd.cpu())
    Vh.copy_(Vd.cpu())
    idx, ns, o = ck.ckv_select_attn(qd, mud, offd, tokd, C, B, Kd, Vd)
    hidx, hns, ho = ck.ckv_select_attn(qd, mud, offd, tokd, C, B, Kh, Vh)
    so = ck.ckv_sparse_attn(qd, Kh, Vh, idx, ns)
    torch.cuda.synchronize()
    assert torch.equal(hidx, idx) and torch.equal(hns, ns)
    assert torch.equal(ho, o) and torch.equal(so, o)

    Kp, Vp = Kd.cpu(), Vd.cpu()                       # pageable
    assert not Kp.is_pinned()
    with pytest.raises(ck.CKVError):
        ck.ckv_select_attn(qd, mud, offd, tokd, C, B, Kp, Vp)
    with pytest.raises(ck.CKVError):
        ck.ckv_sparse_attn(qd, Kp, Vp, idx, ns)
    lib = ck.load()
    sd = ck.SelectDesc(H=H, G=G, d=D, C=C, c_cap=C, n_sink=n_sink, t_cap=tokd.shape[1],
                       pending_begin=0, n_pending=0, B=B, dtype=ck.CKV_BF16)
    ad = ck.AttnDesc(H=H, G=G, d=D, B=B, kv_head_stride=Kd.stride(0), kv_rows=L, scale=0.0,
                     dtype=ck.CKV_BF16)
    ws = torch.empty(ck.ckv_select_attn_workspace(sd, ad), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(o)
    p = lambda t: ct.c_void_p(t.data_ptr())
    st = lib.ckv_select_attn(ct.byref(sd), ct.byref(ad), p(qd), p(mud), p(offd), p(tokd), p(Kp),
                             p(Vp), p(idx), p(ns), p(out), p(ws), ws.numel(),
                             ct.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == ck.CKV_ERR_INVALID_ARG
    wa = torch.empty(ck.ckv_attn_workspace(ad), dtype=torch.uint8, device=DEV)
    st = lib.ckv_sparse_attn(ct.byref(ad), p(qd), p(Kp), p(Vp), p(idx), p(ns), p(out), p(wa),
                             wa.numel(), ct.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == ck.CKV_ERR_INVALID_ARG
    torch.cuda.synchronize()


@pytest.mark.parametrize("L,C,dtype,metric,token_base", [
    (2064, 25, "bf16", "cosine", 0), (2064, 25, "bf16", "l2", 100), (336, 4, "bf16", "cosine", 7),
    (336, 4, "bf16", "inner_product", 0), (2064, 25, "fp32", "cosine", 3)])
def test_cluster_reads_pinned_host_keys_and_refuses_pageable(L, C, dtype, metric, token_base):
    """ckv_cluster over pinned host keys (copied once to the workspace, the
    assignment and the update then reading that copy) equals the clustering
    of the same keys in device memory, on the general and the small-window
    path, for every distance and a nonzero token base; neither call writes
    past the workspace size it declares (the device-key size for device
    keys); a pageable host pointer is refused by the C entry point before
    anything is launched."""
    say(f"ckv_cluster over pinned host keys: L={L} C={C} {dtype} {metric} base={token_base}")
    wl = synth.workload(1 if dtype == "bf16" else 0)
    K, _, _ = synth.make_kv(wl, L=L, heads=range(2)) if dtype == "bf16" else synth.make_kv(wl, L=L)
    Kd = to_dev(K, dtype)
    H = Kd.shape[0]
    m = {"cosine": ck.CKV_COSINE, "inner_product": ck.CKV_INNER_PRODUCT, "l2": ck.CKV_L2}[metric]
    ref = gpu_cluster(Kd, 16, C, 3, token_base=token_base, metric=m)
    Kh = torch.empty(Kd.shape, dtype=Kd.dtype, pin_memory=True)
    Kh.copy_(Kd.cpu())
    outs = [torch.empty_like(x) for x in ref]
    desc = ck.ClusterDesc(H=H, d=D, L=Kd.shape[1], k_head_stride=Kd.stride(0),
                          token_base=token_base, n_sink=16, C=C, iters=3,
                          dtype=ck.CKV_BF16 if dtype == "bf16" else ck.CKV_F32, c_base=0, c_cap=C,
                          t_base=0, t_cap=Kd.shape[1] - 16, metric=m)
    lib = ck.load()
    need = ck.ckv_cluster_workspace(desc)
    guard = 4096                                  # bytes past the declared size, never written
    ws = torch.empty(need + guard, dtype=torch.uint8, device=DEV)
    ws[need:] = 0xA5
    p = lambda t: ct.c_void_p(t.data_ptr())
    stream = ct.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.ckv_cluster(ct.byref(desc), p(Kh), *(p(x) for x in outs), p(ws), need, stream)
    torch.cuda.synchronize()
    assert st == ck.CKV_OK
    for a, b in zip(outs, ref):
        assert torch.equal(a, b)
    assert bool((ws[need:] == 0xA5).all())
    # host keys need the workspace's copy region; device keys do without it
    # and write nothing past the smaller size
    need_dev = ck.ckv_cluster_workspace_device(desc)
    assert 0 < need_dev < need
    st = lib.ckv_cluster(ct.byref(desc), p(Kh), *(p(x) for x in outs), p(ws), need_dev, stream)
    assert st == ck.CKV_ERR_WORKSPACE
    ws[need_dev:] = 0x5A
    outs2 = [torch.empty_like(x) for x in ref]
    st = lib.ckv_cluster(ct.byref(desc), p(Kd), *(p(x) for x in outs2), p(ws), need_dev, stream)
    torch.cuda.synchronize()
    assert st == ck.CKV_OK
    for a, b in zip(outs2, ref):
        assert torch.equal(a, b)
    assert bool((ws[need_dev:] == 0x5A).all())
    Kp = Kd.cpu()
    assert not Kp.is_pinned()
    st = lib.ckv_cluster(ct.byref(desc), p(Kp), *(p(x) for x in outs), p(ws), ws.numel(), stream)
    assert st == ck.CKV_ERR_INVALID_ARG
    torch.cuda.synchronize()
