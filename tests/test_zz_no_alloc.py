"""The allocation-free decode step (ckv_select_attn_noalloc) against
ckv_select_attn.

The caller that cannot allocate (graph capture, serving loops) gets the same
decode step with the library's static per-GPU scratch as workspace. Both
calls run the same kernels, so idx, n_sel and o must be bitwise equal; two
calls in a row share the scratch, the second on a smaller step, and each
must match. A step whose workspace exceeds the scratch, and missing
pointers, return their status before anything is enqueued (host checks).
"""
import ctypes as ct

import numpy as np
import pytest
import torch

import sparse_decode_attention_ckv_amd as ck
import synth
from tests.gpu_helpers import DEV, say, to_dev


def _descs(H, G, C, B, c_cap, t_cap, rows, dtype=ck.CKV_BF16):
    sd = ck.SelectDesc(H=H, G=G, d=128, C=C, c_cap=c_cap, n_sink=16, t_cap=t_cap,
                       pending_begin=0, n_pending=0, B=B, dtype=dtype)
    ad = ck.AttnDesc(H=H, G=G, d=128, B=B, kv_head_stride=rows * 128, kv_rows=rows, scale=0.0,
                     dtype=dtype)
    return sd, ad


def test_noalloc_host_checks():
    lib = ck.load()
    nul = [None] * 9
    # a batched step whose scores and partials exceed the scratch
    sd, ad = _descs(4096, 4, 409, 2048, 409, 32752, 32768)
    assert ck.ckv_select_attn_workspace(sd, ad) > ck.CKV_NOALLOC_SCRATCH_BYTES
    assert lib.ckv_select_attn_noalloc(ct.byref(sd), ct.byref(ad), *nul, None) == \
        ck.CKV_ERR_WORKSPACE
    # a step that fits, with missing pointers
    sd, ad = _descs(8, 4, 409, 1024, 409, 32752, 32768)
    assert ck.ckv_select_attn_workspace(sd, ad) <= ck.CKV_NOALLOC_SCRATCH_BYTES
    assert lib.ckv_select_attn_noalloc(ct.byref(sd), ct.byref(ad), *nul, None) == \
        ck.CKV_ERR_INVALID_ARG
    # the workloads' decode steps fit
    for H, C, B in ((8, 409, 1024), (64, 409, 2048), (8, 1638, 2048), (8, 421, 1024)):
        sd, ad = _descs(H, 4, C, B, C, 131072, 131072)
        assert ck.ckv_select_attn_workspace(sd, ad) <= ck.CKV_NOALLOC_SCRATCH_BYTES, (H, C, B)


@pytest.mark.gpu
def test_noalloc_matches_select_attn_twice():
    wl = synth.workload(1)
    for H, L, C, B in ((8, 8208, 101, 1536), (3, 2064, 25, 256)):
        say(f"noalloc decode step: H={H} L={L} C={C} B={B}")
        K, V, _ = synth.make_kv(wl, L=L, heads=range(H))
        Kd, Vd = to_dev(K, "bf16"), to_dev(V, "bf16")
        qs, _ = synth.make_queries(wl, 3, heads=range(H))
        qd = to_dev(qs, "bf16")
        cent, _, off, tok = ck.ckv_cluster(Kd, 16, C, 4)
        ref = ck.ckv_select_attn(qd, cent, off, tok, C, B, Kd, Vd)
        idx = torch.full((H, B), -7, dtype=torch.int32, device=DEV)
        ns = torch.full((H,), -7, dtype=torch.int32, device=DEV)
        out = torch.full((H * wl.G, 128), float("nan"), dtype=torch.float32, device=DEV)
        got = ck.ckv_select_attn_noalloc(qd, cent, off, tok, C, B, Kd, Vd, idx=idx, n_sel=ns,
                                         out=out)
        torch.cuda.synchronize()
        for x, y in zip(got, ref):
            assert torch.equal(x, y), (H, L, C, B)


@pytest.mark.gpu
def test_noalloc_matches_select_attn_fp32():
    """fp32 rows run the fused fp32 kernel (fp64 attention) in both calls."""
    wl = synth.workload(0)
    for L, C, B in ((2048, 25, 256), (1040, 13, 128)):
        say(f"noalloc decode step, fp32: L={L} C={C} B={B}")
        K, V, _ = synth.make_kv(wl, L=L)
        Kd, Vd = to_dev(K, "f32"), to_dev(V, "f32")
        qs, _ = synth.make_queries(wl, 0)
        qd = to_dev(qs, "f32")
        cent, _, off, tok = ck.ckv_cluster(Kd, 16, C, 4)
        ref = ck.ckv_select_attn(qd, cent, off, tok, C, B, Kd, Vd)
        idx = torch.full((wl.H, B), -7, dtype=torch.int32, device=DEV)
        ns = torch.full((wl.H,), -7, dtype=torch.int32, device=DEV)
        out = torch.full((wl.H * wl.G, 128), float("nan"), dtype=torch.float32, device=DEV)
        got = ck.ckv_select_attn_noalloc(qd, cent, off, tok, C, B, Kd, Vd, idx=idx, n_sel=ns,
                                         out=out)
        torch.cuda.synchronize()
        for x, y in zip(got, ref):
            assert torch.equal(x, y), (L, C, B)
