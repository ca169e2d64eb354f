"""Every entry point writes only inside the buffers it is given (GPU).

Each output is a view into a larger buffer whose bytes before and after the
view hold a pattern, and each workspace is followed by guard bytes past the
size the call declares (the binding hands the library the declared size, not
the tensor's): after the call every pattern byte must still be there. The
shapes are ragged on purpose (and C = 700 takes the three-launch counting
sort and two LDS rounds of centroids): token counts that are not a multiple of
any tile, a budget B that is not a multiple of the 64-row attention split, and
decode rows from pending tokens. ckv_select_attn_noalloc is covered too (its
outputs; its workspace is the library's own), and ckv_cache_step's state.
"""
import numpy as np
import pytest
import torch

import sparse_decode_attention_ckv_amd as ck
import synth
from tests.gpu_helpers import DEV, say, to_dev

pytestmark = pytest.mark.gpu

PAD = 4096                      # pattern bytes on each side (a 16-byte multiple)
PATTERN = 0xA5


class Guarded:
    """A tensor of `shape` with PAD pattern bytes on both sides."""

    def __init__(self, shape, dtype):
        self.n = int(np.prod(shape))
        self.es = torch.empty(0, dtype=dtype).element_size()
        self.pre = PAD // self.es
        self.buf = torch.empty(self.pre + self.n + PAD // self.es, dtype=dtype, device=DEV)
        self.buf.view(torch.uint8).fill_(PATTERN)
        self.t = self.buf[self.pre:self.pre + self.n].view(shape)

    def intact(self) -> bool:
        b = self.buf.view(torch.uint8)
        lo, hi = self.pre * self.es, (self.pre + self.n) * self.es
        return bool((b[:lo] == PATTERN).all()) and bool((b[hi:] == PATTERN).all())


def _guarded_ws(nbytes):
    ws = torch.empty(nbytes + PAD, dtype=torch.uint8, device=DEV)
    ws.fill_(PATTERN)
    return ws


def _ws_intact(ws, nbytes) -> bool:
    return bool((ws[nbytes:] == PATTERN).all())


@pytest.mark.parametrize("H,L,C,dtype,metric", [
    (2, 4121, 51, "bf16", ck.CKV_COSINE), (3, 333, 4, "bf16", ck.CKV_COSINE),
    (1, 2087, 26, "fp32", ck.CKV_COSINE), (2, 6163, 700, "bf16", ck.CKV_COSINE),
    (2, 4121, 51, "bf16", ck.CKV_L2), (1, 2087, 26, "fp32", ck.CKV_INNER_PRODUCT)])
def test_cluster_writes_stay_inside(H, L, C, dtype, metric):
    say(f"bounds: ckv_cluster H={H} L={L} C={C} {dtype} metric={metric}")
    wl = synth.workload(1 if dtype == "bf16" else 0)
    K, _, _ = (synth.make_kv(wl, L=L, heads=range(H)) if dtype == "bf16"
               else synth.make_kv(wl, L=L))
    Kd = to_dev(K, dtype)
    n_sink, Lp = 16, L - 16
    cent = Guarded((H, C, 128), torch.float32)
    asg = Guarded((H, L), torch.int32)
    off = Guarded((H, C + 1), torch.int32)
    tok = Guarded((H, Lp), torch.int32)
    desc = ck.ClusterDesc(H=H, d=128, L=L, k_head_stride=Kd.stride(0), token_base=0,
                          n_sink=n_sink, C=C, iters=4,
                          dtype=ck.CKV_BF16 if dtype == "bf16" else ck.CKV_F32, c_base=0,
                          c_cap=C, t_base=0, t_cap=Lp, metric=metric)
    nb = ck.ckv_cluster_workspace_device(desc)
    ws = _guarded_ws(nb)
    ck.ckv_cluster(Kd, n_sink, C, 4, centroids=cent.t, assign=asg.t, csr_offsets=off.t,
                   csr_tokens=tok.t, workspace=ws, metric=metric)
    torch.cuda.synchronize()
    for name, g in (("centroids", cent), ("assign", asg), ("offsets", off), ("tokens", tok)):
        assert g.intact(), name
    assert _ws_intact(ws, nb)
    # and the results are the ones an unguarded call gives
    ref = ck.ckv_cluster(Kd, n_sink, C, 4, metric=metric)
    torch.cuda.synchronize()
    for a, b in zip((cent.t, asg.t, off.t, tok.t), ref):
        assert torch.equal(a, b)


@pytest.mark.parametrize("G,B,n_pending", [(4, 200, 0), (2, 1000, 37), (1, 65, 3)])
def test_decode_writes_stay_inside(G, B, n_pending):
    say(f"bounds: selection and attention G={G} B={B} pending={n_pending}")
    H, L, C, n_sink = 2, 4121, 51, 16
    wl = synth.workload(1)
    K, V, _ = synth.make_kv(wl, L=L, heads=range(H))
    Kd, Vd = to_dev(K, "bf16"), to_dev(V, "bf16")
    rows = L + n_pending
    Kx = torch.zeros((H, rows, 128), dtype=torch.bfloat16, device=DEV)
    Vx = torch.zeros_like(Kx)
    Kx[:, :L], Vx[:, :L] = Kd, Vd
    Kx[:, L:] = Kd[:, :n_pending]
    Vx[:, L:] = Vd[:, :n_pending]
    cent, _, off, tok = ck.ckv_cluster(Kd, n_sink, C, 3)
    torch.manual_seed(5)
    q = (torch.randn((H * G, 128), device=DEV) * 0.5).to(torch.bfloat16)
    kw = dict(n_sink=n_sink, pending_begin=L, n_pending=n_pending)

    idx = Guarded((H, B), torch.int32)
    nsel = Guarded((H,), torch.int32)
    ck.ckv_select(q, cent, off, tok, C, B, idx=idx.t, n_sel=nsel.t, **kw)
    torch.cuda.synchronize()
    assert idx.intact() and nsel.intact()

    out = Guarded((H * G, 128), torch.float32)
    ck.ckv_sparse_attn(q, Kx, Vx, idx.t, nsel.t, out=out.t)
    torch.cuda.synchronize()
    assert out.intact()

    sd = ck.SelectDesc(H=H, G=G, d=128, C=C, c_cap=C, n_sink=n_sink, t_cap=tok.shape[1],
                       pending_begin=L, n_pending=n_pending, B=B, dtype=ck.CKV_BF16)
    ad = ck.AttnDesc(H=H, G=G, d=128, B=B, kv_head_stride=Kx.stride(0), kv_rows=rows, scale=0.0,
                     dtype=ck.CKV_BF16)
    nb = ck.ckv_select_attn_workspace(sd, ad)
    ws = _guarded_ws(nb)
    idx2 = Guarded((H, B), torch.int32)
    nsel2 = Guarded((H,), torch.int32)
    out2 = Guarded((H * G, 128), torch.float32)
    ck.ckv_select_attn(q, cent, off, tok, C, B, Kx, Vx, idx=idx2.t, n_sel=nsel2.t, out=out2.t,
                       workspace=ws, **kw)
    torch.cuda.synchronize()
    assert idx2.intact() and nsel2.intact() and out2.intact()
    assert _ws_intact(ws, nb)
    # the fused call is bitwise the separate ones
    assert torch.equal(idx2.t, idx.t) and torch.equal(nsel2.t, nsel.t)
    assert torch.equal(out2.t, out.t)

    # the entry point without allocation (its workspace is the library's own)
    idx3 = Guarded((H, B), torch.int32)
    nsel3 = Guarded((H,), torch.int32)
    out3 = Guarded((H * G, 128), torch.float32)
    ck.ckv_select_attn_noalloc(q, cent, off, tok, C, B, Kx, Vx, idx=idx3.t, n_sel=nsel3.t,
                               out=out3.t, **kw)
    torch.cuda.synchronize()
    assert idx3.intact() and nsel3.intact() and out3.intact()
    assert torch.equal(idx3.t, idx.t) and torch.equal(out3.t, out.t)


def test_cache_step_writes_stay_inside():
    """ckv_cache_step: the ring, both row buffers, slot tokens, idx_cache,
    stats and the workspace (a view of exactly the declared size) are guarded
    views; four steps, and the state matches an unguarded run's bitwise."""
    say("bounds: ckv_cache_step, 4 steps")
    H, L, C, n_sink, B, R, G = 2, 4121, 51, 16, 200, 2, 4
    wl = synth.workload(1)
    K, V, _ = synth.make_kv(wl, L=L, heads=range(H))
    Kd, Vd = to_dev(K, "bf16"), to_dev(V, "bf16")
    cent, asg, off, tok = ck.ckv_cluster(Kd, n_sink, C, 3)
    desc = ck.cache_desc(Kd, asg, off, tok, C, B, R, n_sink=n_sink)
    ref = ck.cache_state(desc, DEV)
    guards, st = {}, {"rows": ref["rows"]}
    for k, v in ref.items():
        if isinstance(v, torch.Tensor):
            g = Guarded(tuple(v.shape), v.dtype)
            if k != "workspace":
                g.t.copy_(v)
            guards[k], st[k] = g, g.t
    torch.manual_seed(9)
    for t in range(4):
        q = (torch.randn((H * G, 128), device=DEV) * 0.5).to(torch.bfloat16)
        idx, ns = ck.ckv_select(q, cent, off, tok, C, B, n_sink=n_sink)
        ck.ckv_cache_step(desc, t, idx, ns, asg, off, tok, Kd, Vd, st)
        ck.ckv_cache_step(desc, t, idx, ns, asg, off, tok, Kd, Vd, ref)
    torch.cuda.synchronize()
    for k, g in guards.items():
        assert g.intact(), k
    for k in ("ring", "cache_K", "cache_V", "cache_tok", "idx_cache", "stats"):
        assert torch.equal(st[k], ref[k]), k


@pytest.mark.parametrize("Lw,C", [(320, 4), (1500, 40)])
def test_append_writes_only_its_window(Lw, C):
    """A decode-time increment (c_base, t_base > 0) on the small-window and the
    general path writes centroid rows c_base .. c_base + C - 1, offsets
    c_base .. c_base + C and token slots t_base .. t_base + Lw - 1 of the
    shared buffers, and nothing else of them."""
    say(f"bounds: append window Lw={Lw} C={C}")
    H, L0, c_base, t_base = 2, 2000, 7, 100
    c_cap, t_cap = c_base + C + 5, t_base + Lw + 50
    wl = synth.workload(1)
    K, _, _ = synth.make_kv(wl, L=L0 + Lw, heads=range(H))
    Kd = to_dev(K, "bf16")
    cent = Guarded((H, c_cap, 128), torch.float32)
    off = Guarded((H, c_cap + 1), torch.int32)
    tok = Guarded((H, t_cap), torch.int32)
    asg = Guarded((H, Lw), torch.int32)
    ck.ckv_cluster(Kd[:, L0:], 0, C, 3, token_base=L0, centroids=cent.t, assign=asg.t,
                   csr_offsets=off.t, csr_tokens=tok.t, c_base=c_base, t_base=t_base)
    torch.cuda.synchronize()
    for g in (cent, off, tok, asg):
        assert g.intact()
    pat = lambda x: bool((x.contiguous().view(torch.uint8) == PATTERN).all())
    assert pat(cent.t[:, :c_base]) and pat(cent.t[:, c_base + C:])
    assert pat(off.t[:, :c_base]) and pat(off.t[:, c_base + C + 1:])
    assert pat(tok.t[:, :t_base]) and pat(tok.t[:, t_base + Lw:])
    # the window itself: offsets from t_base to t_base + Lw, every token once
    o = off.t[:, c_base:c_base + C + 1].cpu().numpy()
    assert (o[:, 0] == t_base).all() and (o[:, -1] == t_base + Lw).all()
    w = np.sort(tok.t[:, t_base:t_base + Lw].cpu().numpy(), axis=1)
    assert (w == np.arange(L0, L0 + Lw)[None, :]).all()
