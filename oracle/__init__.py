"""CPU oracle for cluster-granular KV selection -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never does, and this
package never imports the GPU library: the two share no code.

The arithmetic lives in ``ckv_oracle.c`` (plain single-threaded C, fp64),
built with gcc into ``libckv_oracle.so`` next to it. This module only
marshals numpy arrays through ctypes. The GPU cache of selected rows is pure
bookkeeping and is stated in numpy in ``cache.py``. Each wrapper names the page section its
C function follows; the definitions are documented in the C source.

Parity status: every function here is pinned by CPU tests against closed
forms, brute force, textbook routines or invariants (tests/test_oracle_*.py).
"""
from __future__ import annotations

import ctypes as ct
import os
import subprocess

import numpy as np

EXACT = 0
MIRROR = 1

# assignment distances (the page keeps the cosine; the other two are its
# ablation)
COSINE = 0
INNER_PRODUCT = 1
L2 = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ckv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libckv_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (contraction off so that every fused
    multiply-add is an explicit fma() call)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_D = ct.POINTER(ct.c_double)
_I32 = ct.POINTER(ct.c_int32)
_I64 = ct.POINTER(ct.c_int64)
_i64 = ct.c_int64
_int = ct.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ct.CDLL(_LIB_PATH)
    sig = {
        "orc_bf16_round_value": (ct.c_double, [ct.c_double]),
        "orc_unit_rows": (None, [_i64, _int, _D, _int, _D]),
        "orc_init_centroids": (None, [_i64, _int, _D, _int, _int, _D]),
        "orc_assign": (None, [_i64, _int, _D, _int, _int, _D, _int, _I32, _D]),
        "orc_assign_metric": (None, [_i64, _int, _D, _int, _int, _D, _int, _int, _I32, _D]),
        "orc_csr": (None, [_i64, _int, _int, _I32, _i64, _I32, _I32]),
        "orc_update": (None, [_i64, _int, _D, _int, _int, _I32, _D, _int, _D]),
        "orc_objective": (ct.c_double, [_i64, _int, _D, _int, _I32, _D]),
        "orc_cluster": (None, [_int, _int, _i64, _int, _D, _int, _int, _int, _i64,
                               _D, _I32, _I32, _I32, _D, _I64]),
        "orc_cluster_metric": (None, [_int, _int, _int, _i64, _int, _D, _int, _int, _int,
                                      _i64, _D, _I32, _I32, _I32, _D, _I64]),
        "orc_select": (_int, [_int, _int, _int, _D, _int, _int, _D, _I32, _I32,
                              _i64, _int, _i64, _i64, _int, _I32, _I32, _D]),
        "orc_attn": (None, [_int, _int, _int, _D, _D, _D, _i64, _I32, _I32, _int,
                            ct.c_double, _D]),
        "orc_dense_attn": (None, [_int, _int, _int, _D, _D, _D, _i64, _i64,
                                  ct.c_double, _D]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _d(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_D)


def _i(a, dt=np.int32):
    a = np.ascontiguousarray(a, dtype=dt)
    return a, a.ctypes.data_as(_I32 if dt == np.int32 else _I64)


def _null(t):
    return ct.cast(None, t)


def bf16_round(x: float) -> float:
    """The oracle's own bf16 rounding of one value (fp64 -> fp32 -> bf16)."""
    return _load().orc_bf16_round_value(float(x))


def unit_rows(X, mode=EXACT):
    """Unit rows for the cosine distance [ClusterKV, clustering in semantic
    space, distance D]. X: [n][d]."""
    X, px = _d(X)
    n, d = X.shape
    out = np.empty_like(X)
    _load().orc_unit_rows(n, d, px, mode, out.ctypes.data_as(_D))
    return out


def init_centroids(K, n_sink, C):
    """Evenly spaced initial centroids k_{n_sink + s*c}. K: [L][d]."""
    K, pk = _d(K)
    L, d = K.shape
    mu = np.empty((C, d))
    _load().orc_init_centroids(L, d, pk, n_sink, C, mu.ctypes.data_as(_D))
    return mu


def assign(K, n_sink, mu, mode=MIRROR, metric=COSINE):
    """Assignment step [ClusterKV, clustering in semantic space]: cosine by
    default; INNER_PRODUCT and L2 are the page's ablation. K: [L][d],
    mu: [C][d]. Returns (assign [L] int32, margin [L]); the margin is the
    gap between the best and second-best candidate: in cosine units for the
    cosine (MIRROR scores the key as stored against the rounded unit
    centroid and divides the gap by |k|), the score gap for the inner
    product, the squared-distance gap for L2."""
    K, pk = _d(K)
    mu, pm = _d(mu)
    L, d = K.shape
    C = mu.shape[0]
    a = np.empty(L, dtype=np.int32)
    m = np.empty(L)
    if metric == COSINE:
        _load().orc_assign(L, d, pk, n_sink, C, pm, mode, a.ctypes.data_as(_I32),
                           m.ctypes.data_as(_D))
    else:
        _load().orc_assign_metric(L, d, pk, n_sink, C, pm, metric, mode,
                                  a.ctypes.data_as(_I32), m.ctypes.data_as(_D))
    return a, m


def csr(assign_, n_sink, C, token_base=0):
    """Cluster sizes / prefix sums / label-sorted tokens [ClusterKV,
    selection and indexing, Fig. 8]. Returns (offsets [C+1], tokens [L'])."""
    a, pa = _i(assign_)
    L = a.shape[0]
    off = np.empty(C + 1, dtype=np.int32)
    tok = np.empty(L - n_sink, dtype=np.int32)
    _load().orc_csr(L, n_sink, C, pa, token_base, off.ctypes.data_as(_I32),
                    tok.ctypes.data_as(_I32))
    return off, tok


def update(K, n_sink, assign_, mu_old, mode=MIRROR):
    """Centroid update: mean of the raw keys of each cluster [ClusterKV,
    clustering in semantic space]. Returns mu_new [C][d]."""
    K, pk = _d(K)
    a, pa = _i(assign_)
    mu_old, po = _d(mu_old)
    L, d = K.shape
    C = mu_old.shape[0]
    out = np.empty_like(mu_old)
    _load().orc_update(L, d, pk, n_sink, C, pa, po, mode, out.ctypes.data_as(_D))
    return out


def objective(K, n_sink, assign_, mu):
    """Norm-weighted cosine distance J_w of a partition and its centroids."""
    K, pk = _d(K)
    a, pa = _i(assign_)
    mu, pm = _d(mu)
    L, d = K.shape
    return _load().orc_objective(L, d, pk, n_sink, pa, pm)


def cluster(K, n_sink, C, iters, mode=MIRROR, token_base=0, trace=False, metric=COSINE):
    """Full K-means for H heads. K: [H][L][d] (or [L][d] for one head).
    `metric` picks the assignment distance (the trace is the cosine
    objective, so it needs the cosine).

    Returns dict(mu [H][C][d], assign [H][L], offsets [H][C+1],
    tokens [H][L'], trace [H][2*iters] or None, changed [H][iters])."""
    K = np.asarray(K, dtype=np.float64)
    squeeze = K.ndim == 2
    if squeeze:
        K = K[None]
    K, pk = _d(K)
    H, L, d = K.shape
    Lp = L - n_sink
    mu = np.empty((H, C, d))
    a = np.empty((H, L), dtype=np.int32)
    off = np.empty((H, C + 1), dtype=np.int32)
    tok = np.empty((H, Lp), dtype=np.int32)
    tr = np.empty((H, 2 * iters)) if trace else None
    ch = np.empty((H, iters), dtype=np.int64)
    assert not (trace and metric != COSINE), "the trace is the cosine objective"
    _load().orc_cluster_metric(metric, mode, H, L, d, pk, n_sink, C, iters, token_base,
                               mu.ctypes.data_as(_D), a.ctypes.data_as(_I32),
                               off.ctypes.data_as(_I32), tok.ctypes.data_as(_I32),
                               tr.ctypes.data_as(_D) if trace else _null(_D),
                               ch.ctypes.data_as(_I64))
    out = dict(mu=mu, assign=a, offsets=off, tokens=tok, trace=tr, changed=ch)
    if squeeze:
        out = {k: (v[0] if v is not None else None) for k, v in out.items()}
    return out


def select(q, mu, offsets, tokens, C, n_sink, B, G=1, pending_begin=0,
           n_pending=0):
    """Cluster-granular selection [ClusterKV, cluster-granular selection;
    selection and indexing, Fig. 8].

    q: [H*G][d]; mu: [H][c_stride][d]; offsets: [H][c_stride+1];
    tokens: [H][t_stride]. Returns (idx [H][B], n_sel [H], scores [H][C])."""
    q, pq = _d(q)
    mu, pm = _d(mu)
    H, c_stride, d = mu.shape
    off, po = _i(offsets)
    tok, pt = _i(tokens)
    t_stride = tok.shape[1]
    assert off.shape == (H, c_stride + 1) and q.shape == (H * G, d)
    idx = np.empty((H, B), dtype=np.int32)
    ns = np.empty(H, dtype=np.int32)
    sc = np.empty((H, max(C, 1)))
    rc = _load().orc_select(H, G, d, pq, C, c_stride, pm, po, pt, t_stride,
                            n_sink, pending_begin, n_pending, B,
                            idx.ctypes.data_as(_I32), ns.ctypes.data_as(_I32),
                            sc.ctypes.data_as(_D))
    if rc != 0:
        raise ValueError("budget B smaller than sinks + pending tokens")
    return idx, ns, sc[:, :C]


def attn(q, K, V, idx, n_sel, G=1, scale=0.0):
    """softmax(q K_S^T / sqrt(d)) V_S over the selected rows [ClusterKV,
    long-context inference and KV compression]. K, V: [H][rows][d];
    idx: [H][B]; returns o [H*G][d] (fp64)."""
    K, pk = _d(K)
    V, pv = _d(V)
    q, pq = _d(q)
    ix, pi = _i(idx)
    ns, pn = _i(n_sel)
    H, rows, d = K.shape
    B = ix.shape[1]
    o = np.empty((H * G, d))
    _load().orc_attn(H, G, d, pq, pk, pv, rows, pi, pn, B, scale,
                     o.ctypes.data_as(_D))
    return o


def dense_attn(q, K, V, L=None, G=1, scale=0.0):
    """Dense decode attention over rows 0..L-1 [ClusterKV, LLM inference and
    the KV cache]. Returns o [H*G][d] (fp64)."""
    K, pk = _d(K)
    V, pv = _d(V)
    q, pq = _d(q)
    H, rows, d = K.shape
    L = rows if L is None else L
    o = np.empty((H * G, d))
    _load().orc_dense_attn(H, G, d, pq, pk, pv, rows, L, scale,
                           o.ctypes.data_as(_D))
    return o
