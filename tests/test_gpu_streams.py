"""Calls on a stream other than the current one.

Every entry point takes the HIP stream its kernels run on. When the binding
allocates a workspace or a default output for such a call, the memory must
belong to that stream: a block allocated on the current stream and freed on
return could be handed out again, and overwritten, while the side stream's
kernels are still queued. Here the side stream is kept busy, each call is
queued behind that work, and the current stream immediately allocates and
fills memory; the results must equal, bit for bit, the same calls made on the
current stream.
"""
import numpy as np
import pytest
import torch

import sparse_decode_attention_ckv_amd as ck
import synth
from tests.gpu_helpers import DEV, say, to_dev

pytestmark = pytest.mark.gpu


def _busy(s, a):
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(6):
            a = a @ a
            a = a / a.abs().max()
    return a


def _scribble():
    """Allocate and fill on the current stream (picks up any freed block)."""
    junk = [torch.empty(n, dtype=torch.uint8, device=DEV).fill_(0xA5)
            for n in (1 << 16, 1 << 20, 1 << 22, 1 << 24)]
    return junk


def test_side_stream_calls_match_current_stream():
    wl = synth.workload(1)
    H, L, C, B = 2, 4112, 51, 512
    say(f"side-stream calls: H={H} L={L} C={C} B={B}")
    K, V, _ = synth.make_kv(wl, L=L, heads=range(H))
    Kd, Vd = to_dev(K, "bf16"), to_dev(V, "bf16")
    qs, _ = synth.make_queries(wl, 0, heads=range(H))
    qd = to_dev(qs, "bf16")
    ref_cl = ck.ckv_cluster(Kd, 16, C, 4)
    cent, _, off, tok = ref_cl
    ref_sel = ck.ckv_select(qd, cent, off, tok, C, B)
    ref_att = ck.ckv_sparse_attn(qd, Kd, Vd, *ref_sel)
    ref_sa = ck.ckv_select_attn(qd, cent, off, tok, C, B, Kd, Vd)
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    a = torch.randn(3072, 3072, device=DEV)
    calls = {
        "ckv_cluster": (lambda: ck.ckv_cluster(Kd, 16, C, 4, stream=s), ref_cl),
        "ckv_select": (lambda: ck.ckv_select(qd, cent, off, tok, C, B, stream=s), ref_sel),
        "ckv_sparse_attn": (lambda: (ck.ckv_sparse_attn(qd, Kd, Vd, *ref_sel, stream=s),),
                            (ref_att,)),
        "ckv_select_attn": (lambda: ck.ckv_select_attn(qd, cent, off, tok, C, B, Kd, Vd,
                                                       stream=s), ref_sa),
    }
    for name, (call, ref) in calls.items():
        say(f"  {name} on a busy side stream")
        a = _busy(s, a)
        got = call()
        junk = _scribble()
        s.synchronize()
        torch.cuda.synchronize()
        for x, y in zip(got, ref):
            assert torch.equal(x, y), name
        del junk
