"""Seeded synthetic workloads for cluster-granular KV selection.

This module only draws inputs. It holds none of the selection method's
arithmetic, so both the CPU oracle and the GPU library can be fed from it.

Workload shapes follow the ClusterKV page ("ClusterKV: Manipulating LLM KV
Cache in Semantic Space for Recallable Compression"): keys carry a few
large-magnitude outlier channels (section "Clustering in semantic space",
the argument for cosine distance), the first 16 tokens are attention sinks,
C = L/80 clusters are formed at prefill, and new decode tokens are
clustered every 320 steps into 4 clusters. The efficiency experiments use a
Llama-3.1-8B-shaped layer (32 query heads over 8 KV heads, head dim 128)
at a 32k prompt with 1024 decode steps and a 1024-token budget (section
"Experimental results", item 4).

Recipe (one KV head):

* ``n_dirs`` ground-truth directions, uniform on the unit sphere (normalised
  standard normal vectors).
* Each token picks one direction uniformly at random; its key is
  ``direction * N(4, 0.5) + N(0, 0.3)`` per channel (second argument = std).
* Outlier channels: after drawing, the chosen channels of the key are
  multiplied by 20. The single-head fp32 workload uses channels 7 and 93;
  the multi-head workloads draw 4 channels per head without replacement.
* Values are N(0, 1) with no outliers.
* A query is drawn like a key from its KV head's mixture (outliers included).
* The result is rounded to the workload dtype (fp32, or bf16 by
  round-to-nearest-even).

Random streams come from numpy's PCG64 seeded through ``SeedSequence`` with
the workload's master seed and a per-(head, purpose) key, so every array is
reproducible on any host with the same numpy.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import functools
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "bf16_bits", "bf16_to_f32",
    "KVHead", "make_head", "make_kv", "make_queries", "make_query_steps", "make_appended",
    "make_query_stream", "planted_head",
]

# Purposes of the per-head random streams.
_S_DIRS, _S_KEYS, _S_VALS, _S_OUTL, _S_QUERY, _S_APPEND, _S_APPDIRS, _S_QSTREAM = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload.

    H is the number of independent KV-head problems (batch x KV heads),
    G the query heads per KV head.
    """
    name: str
    H: int
    G: int
    d: int
    L: int
    dtype: str                  # "f32" or "bf16"
    n_dirs: int
    outlier_channels: Optional[Sequence[int]]   # fixed channels, or None
    n_outliers: int             # drawn per head when outlier_channels is None
    n_sink: int
    C: int
    iters: int
    B: int
    steps: int
    seed: int
    # incremental decode clustering (appended tokens)
    append_steps: int = 0
    new_dirs: int = 0
    m_every: int = 0
    c_plus: int = 0

    @property
    def Lp(self) -> int:
        """Number of clustered tokens per head, L - n_sink."""
        return self.L - self.n_sink


def _mk(idx: int, **kw) -> Workload:
    return Workload(seed=20241203 + idx, **kw)


# The five workloads. C = floor((L - 16) / 80), which equals floor(L / 80)
# for every size used here.
WORKLOADS = {
    "single_head_fp32_2k": _mk(
        0, name="single_head_fp32_2k", H=1, G=1, d=128, L=2048, dtype="f32",
        n_dirs=25, outlier_channels=(7, 93), n_outliers=2, n_sink=16, C=25,
        iters=10, B=256, steps=1),
    "llama8b_layer_32k": _mk(
        1, name="llama8b_layer_32k", H=8, G=4, d=128, L=32768, dtype="bf16",
        n_dirs=400, outlier_channels=None, n_outliers=4, n_sink=16, C=409,
        iters=10, B=1024, steps=1024),
    "llama8b_layer_32k_batch8": _mk(
        2, name="llama8b_layer_32k_batch8", H=64, G=4, d=128, L=32768,
        dtype="bf16", n_dirs=400, outlier_channels=None, n_outliers=4,
        n_sink=16, C=409, iters=10, B=2048, steps=256),
    "llama8b_layer_32k_incremental": _mk(
        3, name="llama8b_layer_32k_incremental", H=8, G=4, d=128, L=32768,
        dtype="bf16", n_dirs=400, outlier_channels=None, n_outliers=4,
        n_sink=16, C=409, iters=10, B=1024, steps=1024, append_steps=1024,
        new_dirs=20, m_every=320, c_plus=4),
    "llama8b_layer_128k": _mk(
        4, name="llama8b_layer_128k", H=8, G=4, d=128, L=131072,
        dtype="bf16", n_dirs=1600, outlier_channels=None, n_outliers=4,
        n_sink=16, C=1638, iters=10, B=2048, steps=512),
}
_ORDER = list(WORKLOADS)


def workload(key) -> Workload:
    """Look a workload up by name or by its position (0..4)."""
    if isinstance(key, int):
        return WORKLOADS[_ORDER[key]]
    return WORKLOADS[key]


# ----------------------------------------------------------------- dtype ---

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float values to bfloat16 (nearest, ties to even); return raw bits
    as uint16. Input values must be finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _to_dtype(x: np.ndarray, dtype: str):
    """Return (storage, exact float32 values) for the workload dtype."""
    if dtype == "f32":
        v = np.ascontiguousarray(x, dtype=np.float32)
        return v, v
    if dtype == "bf16":
        b = bf16_bits(x)
        return b, bf16_to_f32(b)
    raise ValueError(dtype)


# ------------------------------------------------------------- sampling ---

def _rng(wl_seed: int, head: int, purpose: int, extra: int = 0):
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([wl_seed, head, purpose, extra])))


def _unit_dirs(rng, n: int, d: int) -> np.ndarray:
    g = rng.standard_normal((n, d))
    return g / np.linalg.norm(g, axis=1, keepdims=True)


@functools.lru_cache(maxsize=256)
def _head_dirs(seed: int, head: int, n: int, d: int) -> np.ndarray:
    return _unit_dirs(_rng(seed, head, _S_DIRS), n, d)


def _draw_keys(rng, dirs: np.ndarray, n: int, outl: np.ndarray,
               amp_mean=4.0, amp_sd=0.5, noise_sd=0.3, gain=20.0):
    d = dirs.shape[1]
    z = rng.integers(0, dirs.shape[0], size=n)
    amp = rng.normal(amp_mean, amp_sd, size=n)
    k = dirs[z] * amp[:, None] + rng.normal(0.0, noise_sd, size=(n, d))
    if len(outl):
        k[:, outl] *= gain
    return k, z


@dataclasses.dataclass
class KVHead:
    """One KV head's draw. ``K``/``V`` are storage arrays (float32, or uint16
    bf16 bits); ``Kf``/``Vf`` are their exact float32 values."""
    K: np.ndarray
    V: np.ndarray
    Kf: np.ndarray
    Vf: np.ndarray
    labels: np.ndarray        # planted direction of each token
    dirs: np.ndarray          # planted directions (float64)
    outliers: np.ndarray      # outlier channels of this head


def _outliers(wl: Workload, head: int) -> np.ndarray:
    if wl.outlier_channels is not None:
        return np.asarray(wl.outlier_channels, dtype=np.int64)
    r = _rng(wl.seed, head, _S_OUTL)
    return np.sort(r.choice(wl.d, size=wl.n_outliers, replace=False))


def make_head(wl: Workload, head: int, L: Optional[int] = None) -> KVHead:
    """Draw keys/values of one KV head (rows 0..L-1 of the prompt)."""
    L = wl.L if L is None else L
    dirs = _head_dirs(wl.seed, head, wl.n_dirs, wl.d)
    outl = _outliers(wl, head)
    k, z = _draw_keys(_rng(wl.seed, head, _S_KEYS), dirs, L, outl)
    v = _rng(wl.seed, head, _S_VALS).standard_normal((L, wl.d))
    Ks, Kf = _to_dtype(k, wl.dtype)
    Vs, Vf = _to_dtype(v, wl.dtype)
    return KVHead(Ks, Vs, Kf, Vf, z.astype(np.int32), dirs, outl)


def make_kv(wl: Workload, L: Optional[int] = None, L_cap: Optional[int] = None,
            heads: Optional[Sequence[int]] = None):
    """Stack the heads into [H][L_cap][d] storage arrays (rows >= L are 0).

    Returns (K, V, heads_list)."""
    L = wl.L if L is None else L
    L_cap = L if L_cap is None else L_cap
    hs = list(range(wl.H)) if heads is None else list(heads)
    st = np.float32 if wl.dtype == "f32" else np.uint16
    K = np.zeros((len(hs), L_cap, wl.d), dtype=st)
    V = np.zeros((len(hs), L_cap, wl.d), dtype=st)
    # every head has its own random streams, so drawing them on several
    # threads gives the same arrays as drawing them one after another
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(hs))) as ex:
        out = list(ex.map(lambda h: make_head(wl, h, L), hs))
    for j, hd in enumerate(out):
        K[j, :L] = hd.K
        V[j, :L] = hd.V
    return K, V, out


def make_queries(wl: Workload, step: int, heads: Optional[Sequence[int]] = None):
    """Queries of one decode step: [len(heads) * G][d], drawn like keys of
    each query head's KV head. Returns (storage, float32 values)."""
    hs = list(range(wl.H)) if heads is None else list(heads)
    rows = []
    for h in hs:
        dirs = _head_dirs(wl.seed, h, wl.n_dirs, wl.d)
        outl = _outliers(wl, h)
        k, _ = _draw_keys(_rng(wl.seed, h, _S_QUERY, step), dirs, wl.G, outl)
        rows.append(k)
    q = np.concatenate(rows, axis=0)
    return _to_dtype(q, wl.dtype)


def make_query_steps(wl: Workload, steps: int, heads: Optional[Sequence[int]] = None):
    """Queries of decode steps 0..steps-1 stacked: ([steps][H*G][d] storage,
    float32 values)."""
    st, fv = zip(*(make_queries(wl, t, heads) for t in range(steps)))
    return np.stack(st), np.stack(fv)


def make_query_stream(wl: Workload, steps: int, rho: float,
                      heads: Optional[Sequence[int]] = None):
    """Queries of a decode stream with step-to-step correlation rho:
    q_0 = x_0 and q_t = rho q_{t-1} + sqrt(1 - rho^2) x_t, where each x_t is
    a fresh query drawn like a key of the query head's KV head (outliers
    included). rho = 0 gives independent queries, rho -> 1 a query that
    barely moves. Returns ([steps][len(heads) * G][d] storage, float32
    values)."""
    hs = list(range(wl.H)) if heads is None else list(heads)
    rows = []
    for h in hs:
        dirs = _head_dirs(wl.seed, h, wl.n_dirs, wl.d)
        outl = _outliers(wl, h)
        r = _rng(wl.seed, h, _S_QSTREAM, int(round(rho * 1e6)))
        x, _ = _draw_keys(r, dirs, steps * wl.G, outl)
        x = x.reshape(steps, wl.G, wl.d)
        q = np.empty_like(x)
        q[0] = x[0]
        c = np.sqrt(max(0.0, 1.0 - rho * rho))
        for t in range(1, steps):
            q[t] = rho * q[t - 1] + c * x[t]
        rows.append(q)
    q = np.concatenate(rows, axis=1)
    st, fv = _to_dtype(q.reshape(-1, wl.d), wl.dtype)
    return st.reshape(steps, len(hs) * wl.G, wl.d), fv.reshape(steps, len(hs) * wl.G, wl.d)


def make_appended(wl: Workload, head: int, n: int):
    """Rows appended during decode for the incremental workload: keys drawn
    from the head's directions plus ``new_dirs`` new ones (uniform over
    all), values N(0, 1). Returns (K storage, V storage, Kf, Vf)."""
    dirs = _head_dirs(wl.seed, head, wl.n_dirs, wl.d)
    if wl.new_dirs:
        dirs = np.concatenate(
            [dirs, _unit_dirs(_rng(wl.seed, head, _S_APPDIRS), wl.new_dirs, wl.d)])
    outl = _outliers(wl, head)
    r = _rng(wl.seed, head, _S_APPEND)
    k, _ = _draw_keys(r, dirs, n, outl)
    v = r.standard_normal((n, wl.d))
    Ks, Kf = _to_dtype(k, wl.dtype)
    Vs, Vf = _to_dtype(v, wl.dtype)
    return Ks, Vs, Kf, Vf


def planted_head(n_dirs: int, L: int, d: int, n_sink: int, seed: int,
                 noise_sd: float = 0.02, outliers=(7, 93), dtype="f32"):
    """Well-separated planted mixture for recovery checks.

    Token ``n_sink + s*c`` (s = floor((L - n_sink) / n_dirs)) is forced to
    direction c, so K-means started from those tokens should recover the
    planted partition exactly. Returns (K storage, Kf, labels)."""
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    dirs = _unit_dirs(r, n_dirs, d)
    z = r.integers(0, n_dirs, size=L)
    s = (L - n_sink) // n_dirs
    for c in range(n_dirs):
        z[n_sink + s * c] = c
    amp = r.normal(4.0, 0.5, size=L)
    k = dirs[z] * amp[:, None] + r.normal(0.0, noise_sd, size=(L, d))
    if len(outliers):
        k[:, list(outliers)] *= 20.0
    Ks, Kf = _to_dtype(k, dtype)
    return Ks, Kf, z.astype(np.int32)
