"""Cluster-granular GPU cache of selected KV rows -- TEST INFRASTRUCTURE ONLY.

Oracle of the cache in "ClusterKV: Manipulating LLM KV Cache in Semantic
Space for Recallable Compression", section 缓存选中Token的KV (caching the KV
of selected tokens), with the system overview of Fig. 5 (KV offloaded to CPU
memory at prefill). The GPU keeps the KV of the tokens selected in the last R
decode steps together with the labels of their clusters. At each step the
selected clusters are compared with the cached ones, and only the KV of
clusters that are not cached is loaded from CPU memory.

Definition written out here (plain numpy, no blocking or reordering):

* After step t the cache holds exactly the rows selected in steps
  t-R+1 .. t. A selection takes every admitted cluster's rows as a prefix of
  its CSR segment (the last one cut short), so the union over those steps is,
  per cluster c, the prefix of length N_c = max of the counts n_c(s) it had
  in those steps.
* Layout (a reading; the page fixes none): slot e < n_sink holds sink token
  e, then the clusters follow in ascending id, cluster c's N_c rows in CSR
  order.
* Rows of step t: the cache after step t-1 held m_c = max over steps
  t-R .. t-1 of c's rows. Rows r < m_c of the current selection are hits,
  rows m_c <= r < n_c are loaded from CPU memory. Sinks are loaded at the
  first step and are hits afterwards; they are not counted in the
  statistics.

Only tests/ may import this module.
"""
from __future__ import annotations

import numpy as np


def counts(idx, n_sel, assign, C, token_base=0):
    """Rows of each cluster in one step's selection: [H][C] int64. idx
    [H][B]; the labels come from assign [H][L] (token id - token_base is the
    row). Sinks (label -1) are not counted."""
    H = idx.shape[0]
    out = np.zeros((H, C), dtype=np.int64)
    for h in range(H):
        toks = idx[h, :n_sel[h]].astype(np.int64)
        lab = assign[h, toks - token_base]
        lab = lab[lab >= 0]
        out[h] = np.bincount(lab, minlength=C)[:C]
    return out


def layout(n, n_sink, offsets, tokens):
    """Slots of a cache holding n[c] rows of every cluster c of one head:
    (token id per slot, first slot of every cluster [C])."""
    C = len(n)
    base = n_sink + np.concatenate([[0], np.cumsum(n)[:-1]]).astype(np.int64)
    tok = [np.arange(n_sink, dtype=np.int64)]
    for c in range(C):
        tok.append(tokens[offsets[c]:offsets[c] + n[c]].astype(np.int64))
    return np.concatenate(tok), base


def step(history, idx, n_sel, assign, offsets, tokens, n_sink, R, token_base=0):
    """One decode step of the cache for all heads.

    history: list of [H][C] count arrays of the previous steps (oldest
    first; only the last R are used). idx, n_sel: this step's selection.
    offsets [H][C+1], tokens [H][...]: the CSR.

    Returns dict(history, cache_tok [H] list of arrays, idx_cache [H][B]
    int32 (-1 past n_sel), stats [H][4] = rows hit, rows loaded, clusters
    hit, clusters selected)."""
    H, B = idx.shape
    C = offsets.shape[1] - 1
    n = counts(idx, n_sel, assign, C, token_base)
    prev = history[-R:]
    m = np.max(np.stack(prev), axis=0) if prev else np.zeros_like(n)
    keep = history[-(R - 1):] if R > 1 else []
    N = np.max(np.stack(keep + [n]), axis=0)
    cache_tok, idx_cache = [], np.full((H, B), -1, dtype=np.int32)
    stats = np.zeros((H, 4), dtype=np.int64)
    for h in range(H):
        tok_h, base = layout(N[h], n_sink, offsets[h], tokens[h])
        cache_tok.append(tok_h)
        slot_of = {int(t): s for s, t in enumerate(tok_h)}
        for e in range(n_sel[h]):
            idx_cache[h, e] = slot_of[int(idx[h, e])]
        sel = n[h] > 0
        stats[h, 0] = np.minimum(n[h], m[h]).sum()
        stats[h, 1] = np.maximum(n[h] - m[h], 0).sum()
        stats[h, 2] = (sel & (m[h] >= n[h])).sum()
        stats[h, 3] = sel.sum()
    return dict(history=(history + [n])[-R:], cache_tok=cache_tok, idx_cache=idx_cache,
                stats=stats)


def sources(history, n_now, n_sink, offsets, tokens, R, first):
    """Where every slot of the new cache of one head comes from: an old
    cache slot (>= 0) or a host row (-1 - token id). history: the previous
    steps' count rows of this head [C] (oldest first); n_now: this step's
    counts [C]; first: no previous step (sinks come from the host)."""
    prev = history[-R:]
    m = np.max(np.stack(prev), axis=0) if prev else np.zeros_like(n_now)
    keep = history[-(R - 1):] if R > 1 else []
    N = np.max(np.stack(keep + [n_now]), axis=0)
    _, old_base = layout(m, n_sink, offsets, tokens)
    src = [(-1 - np.arange(n_sink)) if first else np.arange(n_sink)]
    for c in range(len(N)):
        r = np.arange(N[c])
        host = -1 - tokens[offsets[c] + r].astype(np.int64)
        src.append(np.where(r < m[c], old_base[c] + r, host))
    return np.concatenate(src).astype(np.int64)
