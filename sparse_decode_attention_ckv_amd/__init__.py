"""Python binding of libckv: cluster-granular recallable KV selection on
MI355X (gfx950).

Thin marshalling over the C ABI of ``include/ckv.h``: torch tensors supply
device memory and the current HIP stream; every computation runs in the HIP
kernels of ``libckv.so``. There is no CPU fallback: if the library is not
built, every call raises.

Method: "ClusterKV: Manipulating LLM KV Cache in Semantic Space for
Recallable Compression" -- clustering in semantic space (cosine K-means,
16 sinks, C0 = L/80, decode increments of C+ = 4 clusters every m = 320
tokens), cluster-granular selection (q.mu ranking, whole clusters until the
budget B) and sparse decode attention softmax(q K_S^T / sqrt(d)) V_S.
"""
from __future__ import annotations

import contextlib
import ctypes as ct
import os
from typing import Optional

import torch

__all__ = [
    "CKV_OK", "CKV_ERR_INVALID_ARG", "CKV_ERR_UNSUPPORTED", "CKV_ERR_WORKSPACE",
    "CKV_ERR_LAUNCH", "CKVError", "lib_path", "load", "ClusterDesc", "SelectDesc",
    "AttnDesc", "ckv_cluster", "ckv_select", "ckv_sparse_attn",
    "ckv_cluster_workspace", "ckv_cluster_workspace_device", "ckv_select_workspace",
    "ckv_attn_workspace",
    "ckv_status_string", "ckv_abi_version", "ckv_select_attn", "ckv_select_attn_workspace",
    "ckv_cache_rows", "ckv_cache_workspace", "ckv_cache_step", "ckv_device_view",
    "CacheDesc", "cache_desc", "cache_state", "ckv_select_attn_noalloc",
    "CKV_NOALLOC_SCRATCH_BYTES",
]

CKV_OK, CKV_ERR_INVALID_ARG, CKV_ERR_UNSUPPORTED, CKV_ERR_WORKSPACE, CKV_ERR_LAUNCH = range(5)
CKV_F32, CKV_BF16 = 0, 1
CKV_COSINE, CKV_INNER_PRODUCT, CKV_L2 = 0, 1, 2
CKV_NOALLOC_SCRATCH_BYTES = 8 << 20        # include/ckv.h

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libckv.so")
_lib = None


class CKVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {ckv_status_string(status)} (status {status})")


class ClusterDesc(ct.Structure):
    _fields_ = [("H", ct.c_int32), ("d", ct.c_int32), ("L", ct.c_int64),
                ("k_head_stride", ct.c_int64), ("token_base", ct.c_int64),
                ("n_sink", ct.c_int32), ("C", ct.c_int32), ("iters", ct.c_int32),
                ("dtype", ct.c_int32), ("c_base", ct.c_int32), ("c_cap", ct.c_int32),
                ("t_base", ct.c_int64), ("t_cap", ct.c_int64), ("metric", ct.c_int32)]


class SelectDesc(ct.Structure):
    _fields_ = [("H", ct.c_int32), ("G", ct.c_int32), ("d", ct.c_int32), ("C", ct.c_int32),
                ("c_cap", ct.c_int32), ("n_sink", ct.c_int32), ("t_cap", ct.c_int64),
                ("pending_begin", ct.c_int64), ("n_pending", ct.c_int64),
                ("B", ct.c_int32), ("dtype", ct.c_int32)]


class AttnDesc(ct.Structure):
    _fields_ = [("H", ct.c_int32), ("G", ct.c_int32), ("d", ct.c_int32), ("B", ct.c_int32),
                ("kv_head_stride", ct.c_int64), ("kv_rows", ct.c_int64),
                ("scale", ct.c_float), ("dtype", ct.c_int32)]


class CacheDesc(ct.Structure):
    _fields_ = [("H", ct.c_int32), ("d", ct.c_int32), ("C", ct.c_int32), ("c_cap", ct.c_int32),
                ("n_sink", ct.c_int32), ("B", ct.c_int32), ("R", ct.c_int32),
                ("dtype", ct.c_int32), ("L", ct.c_int64), ("token_base", ct.c_int64),
                ("t_cap", ct.c_int64), ("kv_head_stride", ct.c_int64), ("kv_rows", ct.c_int64)]


_P = ct.c_void_p
_SIGS = {
    "ckv_status_string": (ct.c_char_p, [ct.c_int]),
    "ckv_abi_version": (ct.c_int, []),
    "ckv_cluster_workspace": (ct.c_size_t, [ct.POINTER(ClusterDesc)]),
    "ckv_cluster_workspace_device": (ct.c_size_t, [ct.POINTER(ClusterDesc)]),
    "ckv_cluster": (ct.c_int, [ct.POINTER(ClusterDesc), _P, _P, _P, _P, _P, _P, ct.c_size_t, _P]),
    "ckv_select_workspace": (ct.c_size_t, [ct.POINTER(SelectDesc)]),
    "ckv_select": (ct.c_int, [ct.POINTER(SelectDesc), _P, _P, _P, _P, _P, _P, _P, ct.c_size_t, _P]),
    "ckv_attn_workspace": (ct.c_size_t, [ct.POINTER(AttnDesc)]),
    "ckv_sparse_attn": (ct.c_int, [ct.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P, ct.c_size_t, _P]),
    "ckv_select_attn_workspace": (ct.c_size_t, [ct.POINTER(SelectDesc), ct.POINTER(AttnDesc)]),
    "ckv_select_attn": (ct.c_int, [ct.POINTER(SelectDesc), ct.POINTER(AttnDesc), _P, _P, _P, _P,
                                   _P, _P, _P, _P, _P, _P, ct.c_size_t, _P]),
    "ckv_cache_rows": (ct.c_int64, [ct.POINTER(CacheDesc)]),
    "ckv_cache_workspace": (ct.c_size_t, [ct.POINTER(CacheDesc)]),
    "ckv_cache_step": (ct.c_int, [ct.POINTER(CacheDesc), ct.c_int64, _P, _P, _P, _P, _P, _P, _P,
                                  _P, _P, _P, _P, _P, _P, _P, ct.c_size_t, _P]),
    "ckv_device_view": (ct.c_int, [_P, ct.POINTER(ct.c_void_p)]),
    "ckv_select_attn_noalloc": (ct.c_int, [ct.POINTER(SelectDesc), ct.POINTER(AttnDesc), _P, _P,
                                           _P, _P, _P, _P, _P, _P, _P, _P]),
}


def load():
    """Load libckv.so (built in-tree). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(
            f"{lib_path} is missing: build it with `python -m sparse_decode_attention_ckv_amd.build`"
            " (there is no CPU fallback)")
    lib = ct.CDLL(lib_path)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def ckv_status_string(status: int) -> str:
    return load().ckv_status_string(status).decode()


def ckv_abi_version() -> int:
    return load().ckv_abi_version()


# ------------------------------------------------------------ marshalling --

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return CKV_BF16
    if t.dtype == torch.float32:
        return CKV_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ct.c_void_p(t.data_ptr())


def _stream(stream) -> ct.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ct.c_void_p(stream.cuda_stream)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _on_gpu(**tensors):
    """Every tensor a kernel reads or writes as device memory must live on the
    GPU: a host address handed to a kernel would fault. (K and V of the
    attention may also be pinned host tensors; they go through
    ckv_device_view instead.)"""
    for name, t in tensors.items():
        _need(t is None or t.is_cuda, f"{name} must be a GPU tensor")


def _rows(t: torch.Tensor, name: str):
    """[H][rows][d] tensor with contiguous rows; returns head stride (elements)."""
    _need(t.dim() == 3 and t.stride(2) == 1 and t.stride(1) == t.shape[2],
          f"{name} must be [H][rows][d] with contiguous rows")
    return t.stride(0)


def _check(status: int, where: str):
    if status != CKV_OK:
        raise CKVError(status, where)


def _alloc_on(stream):
    """Allocations a call makes for itself (workspace, default outputs) are
    made on the stream its kernels run on, so that torch's caching allocator
    never hands their memory to another stream while those kernels may still
    use it."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor], stream=None):
    """Caller workspace, a fresh one (on the call's stream), or None when the
    call needs none."""
    if ws is not None:
        _need(ws.is_cuda and ws.numel() * ws.element_size() >= nbytes, "workspace too small")
        return ws
    if nbytes == 0:
        return None
    with _alloc_on(stream):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ calls --

def ckv_cluster_workspace(desc: ClusterDesc) -> int:
    return load().ckv_cluster_workspace(ct.byref(desc))


def ckv_cluster_workspace_device(desc: ClusterDesc) -> int:
    """Workspace bytes for ckv_cluster when K is device memory (no room for
    the copy of host keys)."""
    return load().ckv_cluster_workspace_device(ct.byref(desc))


def ckv_select_workspace(desc: SelectDesc) -> int:
    return load().ckv_select_workspace(ct.byref(desc))


def ckv_attn_workspace(desc: AttnDesc) -> int:
    return load().ckv_attn_workspace(ct.byref(desc))


def ckv_select_attn_workspace(sdesc: SelectDesc, adesc: AttnDesc) -> int:
    return load().ckv_select_attn_workspace(ct.byref(sdesc), ct.byref(adesc))


def ckv_cluster(K: torch.Tensor, n_sink: int, C: int, iters: int, *, token_base: int = 0,
                centroids: Optional[torch.Tensor] = None, assign: Optional[torch.Tensor] = None,
                csr_offsets: Optional[torch.Tensor] = None,
                csr_tokens: Optional[torch.Tensor] = None, c_base: int = 0, t_base: int = 0,
                workspace: Optional[torch.Tensor] = None, stream=None,
                metric: int = CKV_COSINE):
    """Cosine K-means over rows n_sink..L-1 of each head of K [H][L][d]
    (metric CKV_INNER_PRODUCT or CKV_L2: the distance ablation).

    Returns (centroids [H][c_cap][d] fp32, assign [H][L] int32,
    csr_offsets [H][c_cap+1] int32, csr_tokens [H][t_cap] int32). Passing
    existing buffers with c_base / t_base appends a window's clusters to them.
    """
    _on_gpu(K=K, centroids=centroids, assign=assign, csr_offsets=csr_offsets,
            csr_tokens=csr_tokens, workspace=workspace)
    lib = load()
    hs = _rows(K, "K")
    H, L, d = K.shape
    dev = K.device
    Lp = L - n_sink
    with _alloc_on(stream):
        if centroids is None:
            centroids = torch.empty((H, c_base + C, d), dtype=torch.float32, device=dev)
        if csr_offsets is None:
            csr_offsets = torch.empty((H, centroids.shape[1] + 1), dtype=torch.int32, device=dev)
        if csr_tokens is None:
            csr_tokens = torch.empty((H, t_base + Lp), dtype=torch.int32, device=dev)
        if assign is None:
            assign = torch.empty((H, L), dtype=torch.int32, device=dev)
    _need(centroids.dtype == torch.float32 and centroids.is_contiguous()
          and centroids.shape[0] == H and centroids.shape[2] == d, "bad centroids buffer")
    _need(csr_offsets.dtype == torch.int32 and csr_offsets.is_contiguous()
          and csr_offsets.shape == (H, centroids.shape[1] + 1), "bad csr_offsets buffer")
    _need(csr_tokens.dtype == torch.int32 and csr_tokens.is_contiguous()
          and csr_tokens.shape[0] == H, "bad csr_tokens buffer")
    _need(assign.dtype == torch.int32 and assign.is_contiguous() and assign.shape == (H, L),
          "bad assign buffer")
    desc = ClusterDesc(H=H, d=d, L=L, k_head_stride=hs, token_base=token_base, n_sink=n_sink,
                       C=C, iters=iters, dtype=_dtype_code(K), c_base=c_base,
                       c_cap=centroids.shape[1], t_base=t_base, t_cap=csr_tokens.shape[1],
                       metric=metric)
    # device keys need no room for the copy that pinned host keys get
    nb = (lib.ckv_cluster_workspace_device if K.is_cuda else lib.ckv_cluster_workspace)(
        ct.byref(desc))
    if nb == 0:
        # report the reason through the call itself (no launch happens)
        _check(lib.ckv_cluster(ct.byref(desc), _ptr(K), _ptr(centroids), _ptr(assign),
                               _ptr(csr_offsets), _ptr(csr_tokens), None, 0, _stream(stream)),
               "ckv_cluster")
    ws = _workspace(nb, dev, workspace, stream)
    _check(lib.ckv_cluster(ct.byref(desc), _ptr(K), _ptr(centroids), _ptr(assign),
                           _ptr(csr_offsets), _ptr(csr_tokens), _ptr(ws), nb, _stream(stream)),
           "ckv_cluster")
    return centroids, assign, csr_offsets, csr_tokens


def ckv_select(q: torch.Tensor, centroids: torch.Tensor, csr_offsets: torch.Tensor,
               csr_tokens: torch.Tensor, C: int, B: int, *, n_sink: int = 16,
               pending_begin: int = 0, n_pending: int = 0, idx: Optional[torch.Tensor] = None,
               n_sel: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               stream=None):
    """Cluster-granular selection for one decode step.

    q [H*G][d]; centroids [H][c_cap][d] fp32; csr_offsets [H][c_cap+1];
    csr_tokens [H][t_cap]. Returns (idx [H][B] int32, n_sel [H] int32)."""
    _on_gpu(q=q, centroids=centroids, csr_offsets=csr_offsets, csr_tokens=csr_tokens, idx=idx,
            n_sel=n_sel, workspace=workspace)
    lib = load()
    H, c_cap, d = centroids.shape
    _need(q.dim() == 2 and q.is_contiguous() and q.shape[1] == d and q.shape[0] % H == 0,
          "q must be [H*G][d] contiguous")
    _need(centroids.dtype == torch.float32 and centroids.is_contiguous(), "bad centroids")
    _need(csr_offsets.dtype == torch.int32 and csr_offsets.is_contiguous()
          and csr_offsets.shape == (H, c_cap + 1), "bad csr_offsets")
    _need(csr_tokens.dtype == torch.int32 and csr_tokens.is_contiguous()
          and csr_tokens.shape[0] == H, "bad csr_tokens")
    dev = q.device
    with _alloc_on(stream):
        if idx is None:
            idx = torch.empty((H, B), dtype=torch.int32, device=dev)
        if n_sel is None:
            n_sel = torch.empty((H,), dtype=torch.int32, device=dev)
    _need(idx.dtype == torch.int32 and idx.is_contiguous() and idx.shape == (H, B), "bad idx")
    _need(n_sel.dtype == torch.int32 and n_sel.numel() == H, "bad n_sel")
    desc = SelectDesc(H=H, G=q.shape[0] // H, d=d, C=C, c_cap=c_cap, n_sink=n_sink,
                      t_cap=csr_tokens.shape[1], pending_begin=pending_begin,
                      n_pending=n_pending, B=B, dtype=_dtype_code(q))
    nb = lib.ckv_select_workspace(ct.byref(desc))
    ws = _workspace(nb, dev, workspace, stream)
    _check(lib.ckv_select(ct.byref(desc), _ptr(q), _ptr(centroids), _ptr(csr_offsets),
                          _ptr(csr_tokens), _ptr(idx), _ptr(n_sel), _ptr(ws), nb,
                          _stream(stream)), "ckv_select")
    return idx, n_sel


def ckv_device_view(t: torch.Tensor) -> int:
    """Device address of a device tensor or of a pinned host tensor (its
    device mapping); raises for pageable host memory."""
    out = ct.c_void_p()
    _check(load().ckv_device_view(ct.c_void_p(t.data_ptr()), ct.byref(out)), "ckv_device_view")
    return out.value


def _kv_ptr(t: torch.Tensor):
    return ct.c_void_p(t.data_ptr() if t.is_cuda else ckv_device_view(t))


def ckv_sparse_attn(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: torch.Tensor,
                    n_sel: torch.Tensor, *, kv_rows: Optional[int] = None, scale: float = 0.0,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None):
    """softmax(q K_S^T * scale) V_S over rows idx[g][:n_sel[g]] of KV head g.

    q [H*G][d]; K, V [H][rows][d] (same strides; device tensors, or pinned
    host tensors read through their device mapping); idx [H][B]; returns
    o [H*G][d] fp32."""
    _on_gpu(q=q, idx=idx, n_sel=n_sel, out=out, workspace=workspace)
    lib = load()
    hs = _rows(K, "K")
    _need(V.shape == K.shape and V.stride() == K.stride() and V.dtype == K.dtype,
          "V must match K in shape, strides and dtype")
    H, rows, d = K.shape
    _need(q.dim() == 2 and q.is_contiguous() and q.shape[1] == d and q.shape[0] % H == 0
          and q.dtype == K.dtype, "q must be [H*G][d] contiguous, dtype of K")
    _need(idx.dtype == torch.int32 and idx.is_contiguous() and idx.dim() == 2
          and idx.shape[0] == H, "bad idx")
    _need(n_sel.dtype == torch.int32 and n_sel.numel() == H, "bad n_sel")
    G = q.shape[0] // H
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((H * G, d), dtype=torch.float32, device=q.device)
    _need(out.dtype == torch.float32 and out.is_contiguous() and out.shape == (H * G, d),
          "bad out")
    desc = AttnDesc(H=H, G=G, d=d, B=idx.shape[1], kv_head_stride=hs,
                    kv_rows=rows if kv_rows is None else kv_rows, scale=scale,
                    dtype=_dtype_code(K))
    nb = lib.ckv_attn_workspace(ct.byref(desc))
    ws = _workspace(nb, q.device, workspace, stream)
    _check(lib.ckv_sparse_attn(ct.byref(desc), _ptr(q), _kv_ptr(K), _kv_ptr(V), _ptr(idx),
                               _ptr(n_sel), _ptr(out), _ptr(ws), nb, _stream(stream)),
           "ckv_sparse_attn")
    return out


# ------------------------------------------------------------------ cache --

def ckv_cache_rows(desc: CacheDesc) -> int:
    return load().ckv_cache_rows(ct.byref(desc))


def ckv_cache_workspace(desc: CacheDesc) -> int:
    return load().ckv_cache_workspace(ct.byref(desc))


def cache_desc(K_src: torch.Tensor, assign: torch.Tensor, csr_offsets: torch.Tensor,
               csr_tokens: torch.Tensor, C: int, B: int, R: int, *, n_sink: int = 16,
               token_base: int = 0) -> CacheDesc:
    """Descriptor of a cache over K_src [H][rows][d] (device or pinned host)
    for selections of budget B over the CSR and labels of ckv_cluster."""
    hs = _rows(K_src, "K_src")
    H, rows, d = K_src.shape
    return CacheDesc(H=H, d=d, C=C, c_cap=csr_offsets.shape[1] - 1, n_sink=n_sink, B=B, R=R,
                     dtype=_dtype_code(K_src), L=assign.shape[1], token_base=token_base,
                     t_cap=csr_tokens.shape[1], kv_head_stride=hs, kv_rows=rows)


def cache_state(desc: CacheDesc, device) -> dict:
    """Zeroed state and output buffers of a cache: ring, the two row buffers
    of K and V, slot tokens, idx_cache, stats and the workspace."""
    rows = ckv_cache_rows(desc)
    _need(rows > 0, "invalid cache descriptor")
    dt = torch.bfloat16 if desc.dtype == CKV_BF16 else torch.float32
    i32 = dict(dtype=torch.int32, device=device)
    return dict(
        rows=rows,
        ring=torch.zeros((desc.H, desc.c_cap, desc.R), **i32),
        cache_K=torch.zeros((2, desc.H, rows, desc.d), dtype=dt, device=device),
        cache_V=torch.zeros((2, desc.H, rows, desc.d), dtype=dt, device=device),
        cache_tok=torch.full((2, desc.H, rows), -1, **i32),
        idx_cache=torch.full((desc.H, desc.B), -1, **i32),
        stats=torch.zeros((desc.H, 5), **i32),
        workspace=torch.empty(max(ckv_cache_workspace(desc), 1), dtype=torch.uint8,
                              device=device))


def ckv_cache_step(desc: CacheDesc, step: int, idx: torch.Tensor, n_sel: torch.Tensor,
                   assign: torch.Tensor, csr_offsets: torch.Tensor, csr_tokens: torch.Tensor,
                   K_src: torch.Tensor, V_src: torch.Tensor, state: dict, stream=None):
    """One decode step of the cache: buffer step & 1 of state["cache_K"] /
    ["cache_V"] then holds the rows selected in the last R steps and
    state["idx_cache"] the slots of this step's selection. Returns the
    (K, V) views of that buffer."""
    _on_gpu(**{k: v for k, v in state.items() if isinstance(v, torch.Tensor)})
    for t, n in ((idx, "idx"), (n_sel, "n_sel"), (assign, "assign"), (csr_offsets, "csr_offsets"),
                 (csr_tokens, "csr_tokens")):
        _need(t.dtype == torch.int32 and t.is_contiguous() and t.is_cuda, f"bad {n}")
    _need(idx.shape == (desc.H, desc.B) and assign.shape == (desc.H, desc.L), "bad idx or assign")
    _need(V_src.shape == K_src.shape and V_src.stride() == K_src.stride(), "V_src must match K_src")
    ws = state["workspace"]
    _check(load().ckv_cache_step(
        ct.byref(desc), step, _ptr(idx), _ptr(n_sel), _ptr(assign), _ptr(csr_offsets),
        _ptr(csr_tokens), ct.c_void_p(K_src.data_ptr()), ct.c_void_p(V_src.data_ptr()),
        _ptr(state["ring"]), _ptr(state["cache_K"]), _ptr(state["cache_V"]),
        _ptr(state["cache_tok"]), _ptr(state["idx_cache"]), _ptr(state["stats"]), _ptr(ws),
        ws.numel(), _stream(stream)), "ckv_cache_step")
    b = step & 1
    return state["cache_K"][b], state["cache_V"][b]


def ckv_select_attn(q: torch.Tensor, centroids: torch.Tensor, csr_offsets: torch.Tensor,
                    csr_tokens: torch.Tensor, C: int, B: int, K: torch.Tensor, V: torch.Tensor,
                    *, n_sink: int = 16, pending_begin: int = 0, n_pending: int = 0,
                    kv_rows: Optional[int] = None, scale: float = 0.0,
                    idx: Optional[torch.Tensor] = None, n_sel: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None):
    """One decode step: ckv_select then ckv_sparse_attn on its output, fused.

    Arguments as in those two calls. Returns (idx [H][B] int32, n_sel [H]
    int32, o [H*G][d] fp32), bitwise what the separate calls return."""
    _on_gpu(q=q, centroids=centroids, csr_offsets=csr_offsets, csr_tokens=csr_tokens, idx=idx,
            n_sel=n_sel, out=out, workspace=workspace)
    lib = load()
    H, c_cap, d = centroids.shape
    hs = _rows(K, "K")
    _need(V.shape == K.shape and V.stride() == K.stride() and V.dtype == K.dtype,
          "V must match K in shape, strides and dtype")
    _need(K.shape[0] == H and K.shape[2] == d, "K must be [H][rows][d] for the centroids' H, d")
    _need(q.dim() == 2 and q.is_contiguous() and q.shape[1] == d and q.shape[0] % H == 0
          and q.dtype == K.dtype, "q must be [H*G][d] contiguous, dtype of K")
    _need(centroids.dtype == torch.float32 and centroids.is_contiguous(), "bad centroids")
    _need(csr_offsets.dtype == torch.int32 and csr_offsets.is_contiguous()
          and csr_offsets.shape == (H, c_cap + 1), "bad csr_offsets")
    _need(csr_tokens.dtype == torch.int32 and csr_tokens.is_contiguous()
          and csr_tokens.shape[0] == H, "bad csr_tokens")
    G = q.shape[0] // H
    dev = q.device
    with _alloc_on(stream):
        if idx is None:
            idx = torch.empty((H, B), dtype=torch.int32, device=dev)
        if n_sel is None:
            n_sel = torch.empty((H,), dtype=torch.int32, device=dev)
        if out is None:
            out = torch.empty((H * G, d), dtype=torch.float32, device=dev)
    _need(idx.dtype == torch.int32 and idx.is_contiguous() and idx.shape == (H, B), "bad idx")
    _need(n_sel.dtype == torch.int32 and n_sel.numel() == H, "bad n_sel")
    _need(out.dtype == torch.float32 and out.is_contiguous() and out.shape == (H * G, d),
          "bad out")
    sd = SelectDesc(H=H, G=G, d=d, C=C, c_cap=c_cap, n_sink=n_sink, t_cap=csr_tokens.shape[1],
                    pending_begin=pending_begin, n_pending=n_pending, B=B,
                    dtype=_dtype_code(q))
    ad = AttnDesc(H=H, G=G, d=d, B=B, kv_head_stride=hs,
                  kv_rows=K.shape[1] if kv_rows is None else kv_rows, scale=scale,
                  dtype=_dtype_code(K))
    nb = lib.ckv_select_attn_workspace(ct.byref(sd), ct.byref(ad))
    ws = _workspace(nb, dev, workspace, stream)
    _check(lib.ckv_select_attn(ct.byref(sd), ct.byref(ad), _ptr(q), _ptr(centroids),
                               _ptr(csr_offsets), _ptr(csr_tokens), _kv_ptr(K), _kv_ptr(V), _ptr(idx),
                               _ptr(n_sel), _ptr(out), _ptr(ws), nb, _stream(stream)),
           "ckv_select_attn")
    return idx, n_sel, out


def ckv_select_attn_noalloc(q: torch.Tensor, centroids: torch.Tensor, csr_offsets: torch.Tensor,
                            csr_tokens: torch.Tensor, C: int, B: int, K: torch.Tensor,
                            V: torch.Tensor, *, idx: torch.Tensor, n_sel: torch.Tensor,
                            out: torch.Tensor, n_sink: int = 16, pending_begin: int = 0,
                            n_pending: int = 0, kv_rows: Optional[int] = None,
                            scale: float = 0.0, stream=None):
    """ckv_select_attn without any allocation: the workspace is the
    library's static per-GPU scratch (CKV_NOALLOC_SCRATCH_BYTES), and the
    caller passes the outputs idx [H][B] int32, n_sel [H] int32 and out
    [H*G][d] fp32. Calls that may overlap on one GPU must not be made.
    Returns (idx, n_sel, out), bitwise what ckv_select_attn returns."""
    _on_gpu(q=q, centroids=centroids, csr_offsets=csr_offsets, csr_tokens=csr_tokens, idx=idx,
            n_sel=n_sel, out=out)
    lib = load()
    H, c_cap, d = centroids.shape
    hs = _rows(K, "K")
    _need(V.shape == K.shape and V.stride() == K.stride() and V.dtype == K.dtype,
          "V must match K in shape, strides and dtype")
    _need(K.shape[0] == H and K.shape[2] == d, "K must be [H][rows][d] for the centroids' H, d")
    _need(q.dim() == 2 and q.is_contiguous() and q.shape[1] == d and q.shape[0] % H == 0
          and q.dtype == K.dtype, "q must be [H*G][d] contiguous, dtype of K")
    _need(centroids.dtype == torch.float32 and centroids.is_contiguous(), "bad centroids")
    _need(csr_offsets.dtype == torch.int32 and csr_offsets.is_contiguous()
          and csr_offsets.shape == (H, c_cap + 1), "bad csr_offsets")
    _need(csr_tokens.dtype == torch.int32 and csr_tokens.is_contiguous()
          and csr_tokens.shape[0] == H, "bad csr_tokens")
    G = q.shape[0] // H
    _need(idx.dtype == torch.int32 and idx.is_contiguous() and idx.shape == (H, B), "bad idx")
    _need(n_sel.dtype == torch.int32 and n_sel.numel() == H, "bad n_sel")
    _need(out.dtype == torch.float32 and out.is_contiguous() and out.shape == (H * G, d),
          "bad out")
    sd = SelectDesc(H=H, G=G, d=d, C=C, c_cap=c_cap, n_sink=n_sink, t_cap=csr_tokens.shape[1],
                    pending_begin=pending_begin, n_pending=n_pending, B=B,
                    dtype=_dtype_code(q))
    ad = AttnDesc(H=H, G=G, d=d, B=B, kv_head_stride=hs,
                  kv_rows=K.shape[1] if kv_rows is None else kv_rows, scale=scale,
                  dtype=_dtype_code(K))
    _check(lib.ckv_select_attn_noalloc(ct.byref(sd), ct.byref(ad), _ptr(q), _ptr(centroids),
                                       _ptr(csr_offsets), _ptr(csr_tokens), _kv_ptr(K),
                                       _kv_ptr(V), _ptr(idx), _ptr(n_sel), _ptr(out),
                                       _stream(stream)), "ckv_select_attn_noalloc")
    return idx, n_sel, out
