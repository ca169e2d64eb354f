"""Host-only checks of the C ABI (no GPU, no kernel launch).

* libckv.so loads and exports every function include/ckv.h declares;
* the ctypes structures of the binding match the C layout gcc computes
  from the header;
* invalid descriptors, missing pointers and short workspaces return their
  status code before anything is enqueued.
"""
import ctypes as ct
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import sparse_decode_attention_ckv_amd as ck

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ckv.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ckv_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = ck.load()
    names = _declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", ck.lib_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ckv_\w+)", out))
    assert set(names) <= exported


def test_struct_layout_matches_header(tmp_path):
    structs = {"ckv_cluster_desc": ck.ClusterDesc, "ckv_select_desc": ck.SelectDesc,
               "ckv_attn_desc": ck.AttnDesc, "ckv_cache_desc": ck.CacheDesc}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ckv.h"', "int main(void){"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)],
                   check=True)
    got = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    for line in got.splitlines():
        cname, field, val = line.split()
        py = structs[cname]
        want = ct.sizeof(py) if field == "size" else getattr(py, field).offset
        assert int(val) == want, line


def test_status_strings():
    for s in range(5):
        assert ck.ckv_status_string(s)
    assert ck.ckv_status_string(99) == "unknown status"
    assert ck.ckv_abi_version() == 4


def _cl(**kw):
    base = dict(H=2, d=128, L=1000, k_head_stride=1000 * 128, token_base=0, n_sink=16, C=12,
                iters=3, dtype=1, c_base=0, c_cap=12, t_base=0, t_cap=984)
    base.update(kw)
    return ck.ClusterDesc(**base)


FAKE = ct.c_void_p(0x1000)   # never dereferenced: every case fails validation


def _call_cluster(desc, ws_bytes=None, nullK=False):
    lib = ck.load()
    need = lib.ckv_cluster_workspace(ct.byref(desc))
    ws = ws_bytes if ws_bytes is not None else need
    return lib.ckv_cluster(ct.byref(desc), None if nullK else FAKE, FAKE, FAKE, FAKE, FAKE,
                           FAKE if ws else None, ws, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=64), ck.CKV_ERR_UNSUPPORTED),
    (dict(d=0), ck.CKV_ERR_INVALID_ARG),
    (dict(C=0), ck.CKV_ERR_INVALID_ARG),
    (dict(C=985, c_cap=985), ck.CKV_ERR_INVALID_ARG),          # C > L - n_sink
    (dict(L=5000, k_head_stride=5000 * 128, C=2049, c_cap=2049, t_cap=4984),
     ck.CKV_ERR_UNSUPPORTED),
    (dict(iters=0), ck.CKV_ERR_INVALID_ARG),
    (dict(H=65536), ck.CKV_ERR_UNSUPPORTED),
    (dict(n_sink=-1), ck.CKV_ERR_INVALID_ARG),
    (dict(n_sink=1000), ck.CKV_ERR_INVALID_ARG),
    (dict(k_head_stride=1000 * 128 - 1), ck.CKV_ERR_INVALID_ARG),
    (dict(c_cap=11), ck.CKV_ERR_INVALID_ARG),
    (dict(c_base=4, c_cap=15), ck.CKV_ERR_INVALID_ARG),
    (dict(t_cap=983), ck.CKV_ERR_INVALID_ARG),
    (dict(dtype=7), ck.CKV_ERR_INVALID_ARG),
    (dict(H=0), ck.CKV_ERR_INVALID_ARG),
    (dict(token_base=-3), ck.CKV_ERR_INVALID_ARG),
    (dict(metric=3), ck.CKV_ERR_INVALID_ARG),
    (dict(metric=-1), ck.CKV_ERR_INVALID_ARG),
])
def test_cluster_rejects_bad_descriptors(kw, status):
    d = _cl(**kw)
    assert ck.load().ckv_cluster_workspace(ct.byref(d)) == 0
    assert _call_cluster(d, ws_bytes=0) == status


def test_cluster_workspace_and_pointer_checks():
    d = _cl()
    lib = ck.load()
    need = lib.ckv_cluster_workspace(ct.byref(d))
    need_dev = lib.ckv_cluster_workspace_device(ct.byref(d))
    # unit centroids + tile histograms + tile ranks, then the host-key copy
    assert need_dev >= 2 * 64 * 128 * 2 + 2 * 1 * 12 * 4 + 2 * 984 * 4
    assert need - need_dev == 2 * 984 * 128 * 2           # H * L' * d * bf16, 256-aligned
    # below the device-key size: refused before the key pointer is looked at
    assert _call_cluster(d, ws_bytes=need_dev - 1) == ck.CKV_ERR_WORKSPACE
    assert _call_cluster(d, nullK=True) == ck.CKV_ERR_INVALID_ARG
    assert lib.ckv_cluster_workspace_device(ct.byref(_cl(C=0))) == 0


def test_cluster_workspace_device_is_a_prefix():
    """Seeded descriptors of both dtypes and all three distances: the device-key
    workspace is the host-key one less the key copy (the last region,
    H * L' * d elements rounded up to 256 bytes)."""
    rng = np.random.default_rng(11)
    lib = ck.load()
    for _ in range(64):
        H = int(rng.integers(1, 65))
        n_sink = int(rng.integers(0, 33))
        L = n_sink + int(rng.integers(1, 200000))
        C = int(rng.integers(1, min(2048, L - n_sink) + 1))
        dtype = [ck.CKV_BF16, ck.CKV_F32][int(rng.integers(0, 2))]
        d = _cl(H=H, L=L, n_sink=n_sink, C=C, c_cap=C, t_cap=L - n_sink, dtype=dtype,
                metric=int(rng.integers(0, 3)), k_head_stride=L * 128)
        need = lib.ckv_cluster_workspace(ct.byref(d))
        need_dev = lib.ckv_cluster_workspace_device(ct.byref(d))
        es = 2 if dtype == ck.CKV_BF16 else 4
        copy = (H * (L - n_sink) * 128 * es + 255) // 256 * 256
        assert need_dev > 0 and need - need_dev == copy, (H, L, n_sink, C, dtype)


def _sel(**kw):
    base = dict(H=2, G=4, d=128, C=10, c_cap=10, n_sink=16, t_cap=500, pending_begin=0,
                n_pending=0, B=64, dtype=1)
    base.update(kw)
    return ck.SelectDesc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(G=0), ck.CKV_ERR_INVALID_ARG), (dict(G=9), ck.CKV_ERR_INVALID_ARG),
    (dict(d=96), ck.CKV_ERR_UNSUPPORTED), (dict(C=0), ck.CKV_ERR_INVALID_ARG),
    (dict(C=11), ck.CKV_ERR_INVALID_ARG), (dict(B=15), ck.CKV_ERR_INVALID_ARG),
    (dict(n_pending=60), ck.CKV_ERR_INVALID_ARG), (dict(pending_begin=-1), ck.CKV_ERR_INVALID_ARG),
    (dict(C=2049, c_cap=4096), ck.CKV_ERR_UNSUPPORTED), (dict(t_cap=0), ck.CKV_ERR_INVALID_ARG),
    (dict(H=65536), ck.CKV_ERR_UNSUPPORTED),
])
def test_select_rejects_bad_descriptors(kw, status):
    d = _sel(**kw)
    lib = ck.load()
    assert lib.ckv_select_workspace(ct.byref(d)) == 0
    assert lib.ckv_select(ct.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == status


def test_select_workspace_and_pointers():
    d = _sel()
    lib = ck.load()
    need = lib.ckv_select_workspace(ct.byref(d))
    assert need >= 2 * 10 * 8 and need % 256 == 0           # fp64 scores [H][C]
    for k in range(6):                                       # any missing pointer is rejected
        args = [FAKE] * 6
        args[k] = None
        assert lib.ckv_select(ct.byref(d), *args, FAKE, need, None) == ck.CKV_ERR_INVALID_ARG
    d = _sel(C=1000, c_cap=1000, t_cap=5000)
    need = lib.ckv_select_workspace(ct.byref(d))
    assert need >= 2 * 1000 * 8 and need % 256 == 0
    assert lib.ckv_select(ct.byref(d), *[FAKE] * 6, None, need, None) == ck.CKV_ERR_WORKSPACE
    assert lib.ckv_select(ct.byref(d), *[FAKE] * 6, FAKE, need - 1, None) == ck.CKV_ERR_WORKSPACE
    # budgets beyond 2^20 slots per head are not supported
    d = _sel(B=(1 << 20) + 1)
    assert lib.ckv_select_workspace(ct.byref(d)) == 0
    assert lib.ckv_select(ct.byref(d), *[FAKE] * 6, FAKE, 1 << 20, None) == ck.CKV_ERR_UNSUPPORTED


def _att(**kw):
    base = dict(H=2, G=4, d=128, B=64, kv_head_stride=300 * 128, kv_rows=300, scale=0.0, dtype=1)
    base.update(kw)
    return ck.AttnDesc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(G=0), ck.CKV_ERR_INVALID_ARG), (dict(d=256), ck.CKV_ERR_UNSUPPORTED),
    (dict(B=0), ck.CKV_ERR_INVALID_ARG), (dict(kv_rows=0), ck.CKV_ERR_INVALID_ARG),
    (dict(kv_head_stride=100), ck.CKV_ERR_INVALID_ARG), (dict(dtype=2), ck.CKV_ERR_INVALID_ARG),
    (dict(scale=float("nan")), ck.CKV_ERR_INVALID_ARG),
    (dict(B=32769, kv_rows=40000, kv_head_stride=40000 * 128), ck.CKV_ERR_UNSUPPORTED),
    (dict(H=65536), ck.CKV_ERR_UNSUPPORTED),
])
def test_attn_rejects_bad_descriptors(kw, status):
    d = _att(**kw)
    lib = ck.load()
    assert lib.ckv_attn_workspace(ct.byref(d)) == 0
    assert lib.ckv_sparse_attn(ct.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                               None) == status


def test_attn_workspace_and_pointers():
    d = _att()
    lib = ck.load()
    need = lib.ckv_attn_workspace(ct.byref(d))
    assert need >= 2 * 4 * 1 * 130 * 4 + 2 * 4   # one 64-row split per head + counters
    assert lib.ckv_sparse_attn(ct.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                               None) == ck.CKV_ERR_WORKSPACE
    assert lib.ckv_sparse_attn(ct.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, need,
                               None) == ck.CKV_ERR_INVALID_ARG


def test_select_attn_checks():
    lib = ck.load()
    sd, ad = _sel(), _att()
    need = lib.ckv_select_attn_workspace(ct.byref(sd), ct.byref(ad))
    assert need == lib.ckv_select_workspace(ct.byref(sd)) + lib.ckv_attn_workspace(ct.byref(ad))
    args = [FAKE] * 9
    assert lib.ckv_select_attn(ct.byref(sd), ct.byref(ad), *args, FAKE, need - 1,
                               None) == ck.CKV_ERR_WORKSPACE
    for k in range(9):                                      # any missing pointer is rejected
        a = list(args)
        a[k] = None
        assert lib.ckv_select_attn(ct.byref(sd), ct.byref(ad), *a, FAKE, need,
                                   None) == ck.CKV_ERR_INVALID_ARG
    # the two descriptors must describe the same step
    for kw in (dict(H=3), dict(G=2), dict(B=128), dict(dtype=0)):
        sd2 = _sel(**kw)
        assert lib.ckv_select_attn_workspace(ct.byref(sd2), ct.byref(ad)) == 0
        assert lib.ckv_select_attn(ct.byref(sd2), ct.byref(ad), *args, FAKE, need,
                                   None) == ck.CKV_ERR_INVALID_ARG
    # each descriptor is also checked on its own
    assert lib.ckv_select_attn(ct.byref(_sel(d=64)), ct.byref(_att(d=64)), *args, FAKE, need,
                               None) == ck.CKV_ERR_UNSUPPORTED


def _cache(**kw):
    base = dict(H=2, d=128, C=25, c_cap=30, n_sink=16, B=256, R=2, dtype=1, L=2064,
                token_base=0, t_cap=2048, kv_head_stride=2064 * 128, kv_rows=2064)
    base.update(kw)
    return ck.CacheDesc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(d=64), ck.CKV_ERR_UNSUPPORTED),
    (dict(C=0), ck.CKV_ERR_INVALID_ARG),
    (dict(C=31), ck.CKV_ERR_INVALID_ARG),                     # C > c_cap
    (dict(C=2049, c_cap=2049), ck.CKV_ERR_UNSUPPORTED),
    (dict(R=0), ck.CKV_ERR_INVALID_ARG),
    (dict(R=9), ck.CKV_ERR_UNSUPPORTED),
    (dict(B=4097), ck.CKV_ERR_UNSUPPORTED),
    (dict(B=8), ck.CKV_ERR_INVALID_ARG),                      # B < n_sink
    (dict(n_sink=-1), ck.CKV_ERR_INVALID_ARG),
    (dict(kv_head_stride=2064 * 128 - 1), ck.CKV_ERR_INVALID_ARG),
    (dict(kv_rows=0), ck.CKV_ERR_INVALID_ARG),
    (dict(t_cap=0), ck.CKV_ERR_INVALID_ARG),
    (dict(token_base=-1), ck.CKV_ERR_INVALID_ARG),
    (dict(dtype=5), ck.CKV_ERR_INVALID_ARG),
    (dict(H=0), ck.CKV_ERR_INVALID_ARG),
])
def test_cache_rejects_bad_descriptors(kw, status):
    d = _cache(**kw)
    lib = ck.load()
    assert lib.ckv_cache_rows(ct.byref(d)) == 0
    assert lib.ckv_cache_workspace(ct.byref(d)) == 0
    assert lib.ckv_cache_step(ct.byref(d), 0, *([FAKE] * 13), None, 0, None) == status


def test_cache_sizes_and_pointer_checks():
    d = _cache()
    lib = ck.load()
    rows = lib.ckv_cache_rows(ct.byref(d))
    assert rows == 16 + 2 * (256 - 16)
    ws = lib.ckv_cache_workspace(ct.byref(d))
    assert ws >= 2 * rows * 4 + 2 * 4
    ptrs = [FAKE] * 13
    for i in range(13):
        if i in (5, 6):          # K_src / V_src are checked by the device-view step
            continue
        bad = list(ptrs)
        bad[i] = None
        assert lib.ckv_cache_step(ct.byref(d), 0, *bad, FAKE, ws, None) == ck.CKV_ERR_INVALID_ARG
    assert lib.ckv_cache_step(ct.byref(d), -1, *ptrs, FAKE, ws, None) == ck.CKV_ERR_INVALID_ARG
    assert lib.ckv_device_view(FAKE, None) == ck.CKV_ERR_INVALID_ARG


def test_binding_refuses_host_tensors_before_any_call():
    """A CPU tensor where a kernel reads or writes device memory is refused by
    the binding (ValueError) before the library or the GPU is touched."""
    d = 128
    q = torch.zeros(4, d, dtype=torch.bfloat16)
    K = torch.zeros(1, 64, d, dtype=torch.bfloat16)
    cent = torch.zeros(1, 3, d)
    off = torch.zeros(1, 4, dtype=torch.int32)
    tok = torch.zeros(1, 48, dtype=torch.int32)
    idx = torch.zeros(1, 32, dtype=torch.int32)
    ns = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        ck.ckv_cluster(K, 16, 3, 1)
    with pytest.raises(ValueError, match="GPU tensor"):
        ck.ckv_select(q, cent, off, tok, 3, 32)
    with pytest.raises(ValueError, match="GPU tensor"):
        ck.ckv_sparse_attn(q, K, K, idx, ns)
    with pytest.raises(ValueError, match="GPU tensor"):
        ck.ckv_select_attn(q, cent, off, tok, 3, 32, K, K)
