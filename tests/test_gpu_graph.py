"""GPU: calls reusing one workspace, and captured as a HIP graph.

These tests reuse one workspace for many calls and replay a captured decode
loop and a captured clustering call several times (with eager work and
synchronisations between replays), checking every result bitwise against
eager calls.
"""
import numpy as np
import pytest
import torch

import sparse_decode_attention_ckv_amd as ck
import synth
from tests.gpu_helpers import DEV, say, to_dev

pytestmark = pytest.mark.gpu


def _setup(H=8, L=8192, C=101, B=512, steps=6):
    wl = synth.workload(1)
    K, V, _ = synth.make_kv(wl, L=L, heads=range(H))
    Kd, Vd = to_dev(K, "bf16"), to_dev(V, "bf16")
    cent, asg, off, tok = ck.ckv_cluster(Kd, 16, C, 4)
    Q = torch.stack([to_dev(synth.make_queries(wl, t, heads=range(H))[0], "bf16")
                     for t in range(steps)])
    return wl, Kd, Vd, cent, off, tok, Q, C, B


def test_workspace_reused_across_calls():
    say("decode calls reusing one zeroed workspace")
    wl, Kd, Vd, cent, off, tok, Q, C, B = _setup()
    H, G = Kd.shape[0], wl.G
    sd = ck.SelectDesc(H=H, G=G, d=128, C=C, c_cap=C, n_sink=16, t_cap=tok.shape[1],
                       pending_begin=0, n_pending=0, B=B, dtype=ck.CKV_BF16)
    ad = ck.AttnDesc(H=H, G=G, d=128, B=B, kv_head_stride=Kd.stride(0), kv_rows=Kd.shape[1],
                     scale=0.0, dtype=ck.CKV_BF16)
    ws_s = torch.empty(max(ck.ckv_select_workspace(sd), 1), dtype=torch.uint8, device=DEV)
    ws_a = torch.empty(ck.ckv_attn_workspace(ad), dtype=torch.uint8, device=DEV)
    for t in range(Q.shape[0]):
        i1, n1 = ck.ckv_select(Q[t], cent, off, tok, C, B)            # fresh workspace
        o1 = ck.ckv_sparse_attn(Q[t], Kd, Vd, i1, n1)
        for rep in range(3):                                           # reused workspace
            i2, n2 = ck.ckv_select(Q[t], cent, off, tok, C, B, workspace=ws_s)
            o2 = ck.ckv_sparse_attn(Q[t], Kd, Vd, i2, n2, workspace=ws_a)
            torch.cuda.synchronize()
            assert torch.equal(i1, i2) and torch.equal(n1, n2) and torch.equal(o1, o2)


def test_decode_graph_replay_matches_eager():
    say("decode loop captured as a HIP graph, replayed 3 times")
    wl, Kd, Vd, cent, off, tok, Q, C, B = _setup()
    H, G, T = Kd.shape[0], wl.G, Q.shape[0]
    sd = ck.SelectDesc(H=H, G=G, d=128, C=C, c_cap=C, n_sink=16, t_cap=tok.shape[1],
                       pending_begin=0, n_pending=0, B=B, dtype=ck.CKV_BF16)
    ad = ck.AttnDesc(H=H, G=G, d=128, B=B, kv_head_stride=Kd.stride(0), kv_rows=Kd.shape[1],
                     scale=0.0, dtype=ck.CKV_BF16)
    ws_s = torch.empty(max(ck.ckv_select_workspace(sd), 1), dtype=torch.uint8, device=DEV)
    ws_a = torch.empty(ck.ckv_attn_workspace(ad), dtype=torch.uint8, device=DEV)
    idx = torch.full((T, H, B), -7, dtype=torch.int32, device=DEV)
    ns = torch.zeros((T, H), dtype=torch.int32, device=DEV)
    O = torch.zeros((T, H * G, 128), dtype=torch.float32, device=DEV)

    def loop():
        for t in range(T):
            ck.ckv_select(Q[t], cent, off, tok, C, B, idx=idx[t], n_sel=ns[t], workspace=ws_s)
            ck.ckv_sparse_attn(Q[t], Kd, Vd, idx[t], ns[t], out=O[t], workspace=ws_a)

    loop()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (idx, ns, O)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop()
    for rep in range(3):
        idx.fill_(-7)
        O.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (idx, ns, O)):
            assert torch.equal(a, b), rep
        loop()                                                 # eager work between replays
        torch.cuda.synchronize()
        for a, b in zip(ref, (idx, ns, O)):
            assert torch.equal(a, b), rep


@pytest.mark.parametrize("H,L,C", [
    (4, 8192, 101),      # C <= 512: the two-launch CSR over 2048-token tiles
    (2, 12000, 600),     # C > 512: the three-launch CSR, two LDS rounds in the assignment
])
def test_cluster_graph_replay_matches_eager(H, L, C):
    """The whole Lloyd loop (normalisation, initial centroids, 10 x assignment,
    counting sort and update) captured once and replayed 3 times, with eager
    work between the replays: every replay equals the eager call bitwise."""
    say(f"ckv_cluster captured as a HIP graph: H={H} L={L} C={C}, 3 replays")
    wl = synth.workload(1)
    K, _, _ = synth.make_kv(wl, L=L, heads=range(H))
    Kd = to_dev(K, "bf16")
    ref = ck.ckv_cluster(Kd, 16, C, 10)
    torch.cuda.synchronize()
    out = [torch.empty_like(x) for x in ref]
    desc = ck.ClusterDesc(H=H, d=128, L=L, k_head_stride=Kd.stride(0), token_base=0, n_sink=16,
                          C=C, iters=10, dtype=ck.CKV_BF16, c_base=0, c_cap=C, t_base=0,
                          t_cap=L - 16, metric=ck.CKV_COSINE)
    ws = torch.empty(ck.ckv_cluster_workspace_device(desc), dtype=torch.uint8, device=DEV)

    def call():
        ck.ckv_cluster(Kd, 16, C, 10, centroids=out[0], assign=out[1], csr_offsets=out[2],
                       csr_tokens=out[3], workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    junk = torch.empty(1 << 22, dtype=torch.uint8, device=DEV)
    for rep in range(3):
        for x in out:
            x.view(torch.uint8).fill_(0xA5)
        junk.fill_(rep)                                  # eager work between the replays
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, out):
            assert torch.equal(a, b), rep
