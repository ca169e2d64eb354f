"""Pins of the cache oracle (no GPU).

The oracle states the cache by per-cluster row counts (the union of CSR
prefixes is the prefix of the longest). Here every step of a real selection
stream is checked by plain set algebra on token ids instead: the cache holds
exactly the sinks and the tokens selected in the last R steps, each once;
hits and loads are the selected tokens inside and outside the previous
cache; idx_cache addresses the selected tokens; every slot's source holds
the token it claims.
"""
import numpy as np
import pytest

import oracle
from oracle import cache as oc
import synth

N_SINK, C, B, STEPS = 16, 25, 256, 14


@pytest.fixture(scope="module")
def stream():
    wl = synth.workload(1)
    heads = [0, 1]
    K, _, hs = synth.make_kv(wl, L=2064, heads=heads)
    Kf = np.stack([h.Kf for h in hs]).astype(np.float64)
    cl = oracle.cluster(Kf, N_SINK, C, 6)
    _, qf = synth.make_query_stream(wl, STEPS, 0.8, heads=heads)
    sels = []
    for t in range(STEPS):
        idx, ns, _ = oracle.select(qf[t].astype(np.float64), cl["mu"], cl["offsets"],
                                   cl["tokens"], C, N_SINK, B, G=wl.G)
        sels.append((idx, ns))
    return cl, sels


def _set(idx, ns, h):
    return set(int(x) for x in idx[h, :ns[h]]) - set(range(N_SINK))


@pytest.mark.parametrize("R", [1, 2, 3])
def test_cache_is_the_union_of_the_last_R_selections(stream, R):
    cl, sels = stream
    H = sels[0][0].shape[0]
    hist, prev_tok = [], None
    loads = hits = 0
    for t, (idx, ns) in enumerate(sels):
        out = oc.step(hist, idx, ns, cl["assign"], cl["offsets"], cl["tokens"], N_SINK, R)
        for h in range(H):
            tok = out["cache_tok"][h]
            want = set(range(N_SINK))
            for s in range(max(0, t - R + 1), t + 1):
                want |= _set(*sels[s], h)
            assert len(tok) == len(set(tok.tolist())) == len(want)
            assert set(tok.tolist()) == want
            assert len(tok) <= N_SINK + R * (B - N_SINK)
            e = np.arange(ns[h])
            assert np.array_equal(tok[out["idx_cache"][h, e]], idx[h, e])
            assert np.all(out["idx_cache"][h, ns[h]:] == -1)
            now = _set(idx, ns, h)
            before = set() if prev_tok is None else set(prev_tok[h].tolist())
            st = out["stats"][h]
            assert st[0] == len(now & before) and st[1] == len(now - before)
            labels = {}
            for x in now:
                labels.setdefault(int(cl["assign"][h, x]), []).append(x)
            assert st[3] == len(labels)
            assert st[2] == sum(all(x in before for x in v) for v in labels.values())
            hits += st[0]
            loads += st[1]
            # every slot's source holds the token the slot claims
            n_now = oc.counts(idx[h:h + 1], ns[h:h + 1], cl["assign"][h:h + 1], C)[0]
            src = oc.sources([x[h] for x in hist], n_now, N_SINK, cl["offsets"][h],
                             cl["tokens"][h], R, first=(t == 0))
            assert len(src) == len(tok)
            for s, v in enumerate(src):
                if v >= 0:
                    assert prev_tok[h][v] == tok[s]
                else:
                    assert -1 - v == tok[s] and (t == 0 or int(tok[s]) not in before)
            assert (src < 0).sum() == st[1] + (N_SINK if t == 0 else 0)
        hist, prev_tok = out["history"], out["cache_tok"]
    assert hits > 0 and loads > 0


def test_repeated_and_alternating_selections():
    # hand-made CSR: 4 clusters of 5 tokens after 2 sinks
    n_sink = 2
    offsets = np.array([[0, 5, 10, 15, 20]])
    tokens = np.arange(n_sink, n_sink + 20)[None]
    assign = np.array([[-1, -1] + [c for c in range(4) for _ in range(5)]])
    a = np.array([[0, 1, 2, 3, 4, 5, 6, 7, 8, -1, -1]])          # cluster 0 + 2 rows of 1
    b = np.array([[0, 1, 12, 13, 14, 15, 16, 17, 18, -1, -1]])   # cluster 2 + 2 rows of 3
    ns = np.array([9])
    for R, seq, want_hits in [
        (1, [a, a, a], [0, 7, 7]),
        (1, [a, b, a, b], [0, 0, 0, 0]),
        (2, [a, b, a, b], [0, 0, 7, 7]),
    ]:
        hist = []
        for t, sel in enumerate(seq):
            out = oc.step(hist, sel, ns, assign, offsets, tokens, n_sink, R)
            assert out["stats"][0, 0] == want_hits[t], (R, t)
            assert out["stats"][0, 0] + out["stats"][0, 1] == 7
            hist = out["history"]
    # a longer prefix of a cached cluster: only the new rows are loaded
    c1 = np.array([[0, 1, 7, 8, 9, 10, 11, -1, -1, -1, -1]])      # all 5 rows of cluster 1
    hist = oc.step([], a, ns, assign, offsets, tokens, n_sink, 1)["history"]
    out = oc.step(hist, c1, np.array([7]), assign, offsets, tokens, n_sink, 1)
    assert out["stats"][0].tolist() == [2, 3, 0, 1]       # 2 cached rows hit, 3 loaded
