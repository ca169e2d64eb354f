"""Decode-time clustering on a second stream, overlapping decode steps.

The incremental 32k layer (8 KV heads, 1024 decode steps, one new K/V row per
head per step, every 320 steps the newest 320 rows clustered into 4 clusters)
with each increment forked onto a side stream after the step that completes
its rows and joined `lag` steps later. The decode steps in between keep
selecting those rows as pending rows. Checks, in the launch configuration the
benchmark uses (fused select + attention, preallocated workspaces):
  * the overlapped run equals, bit for bit, the same schedule run on one
    stream (so the streams do not race), eagerly, as one replayed HIP graph
    and as the linear graphs joined by events that the benchmark replays;
  * selection at every step equals the oracle's for that step's cluster
    count and pending rows; attention at the steps around every fork and join
    is within 2e-3 of exact fp64 attention over the oracle's rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from sparse_decode_attention_ckv_amd.incremental import IncrementalDecoder, capture
from tests.gpu_helpers import DEV, host_f64, rel_err, say

pytestmark = pytest.mark.gpu


class _Layer:
    """The incremental 32k layer on the GPU: K and V with room for the
    appended rows (decode step t writes row L + t of both first), the steps'
    queries, and the package's IncrementalDecoder over them."""

    def __init__(self, wl):
        T, L, H = wl.append_steps, wl.L, wl.H
        K, V, _ = synth.make_kv(wl, L=L, L_cap=L + T)
        Q, _ = synth.make_query_steps(wl, T)
        app = [synth.make_appended(wl, h, T) for h in range(H)]

        def bf(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(DEV)
        self.wl, self.T = wl, T
        self.KV = bf(np.stack([K, V]))
        self.KVa = bf(np.stack([np.stack([x[0] for x in app]), np.stack([x[1] for x in app])]))
        self.K, self.V, self.Q = self.KV[0], self.KV[1], bf(Q)
        self.dec = IncrementalDecoder(self.K, self.V, self.Q, L=L, n_sink=wl.n_sink, C=wl.C,
                                      iters=wl.iters, B=wl.B, m=wl.m_every, c_plus=wl.c_plus,
                                      before_step=self.append)

    def append(self, t):
        self.KV[:, :, self.wl.L + t].copy_(self.KVa[:, :, t])


@pytest.fixture(scope="module")
def layer():
    wl = synth.workload("llama8b_layer_32k_incremental")
    say(f"async clustering: drawing the {wl.name} inputs")
    return _Layer(wl)


def _run(dec):
    dec.prefill()
    dec.decode()
    torch.cuda.synchronize()
    return dec.snapshot()


@pytest.mark.parametrize("lag", [0, 32, 319])
def test_overlapped_increments_match_one_stream(layer, lag):
    dec, wl, T, m = layer.dec, layer.wl, layer.T, layer.wl.m_every
    side = torch.cuda.Stream(device=DEV)
    say(f"async clustering lag {lag}: one stream")
    dec.set_lag(lag, None)
    ref = _run(dec)
    say(f"async clustering lag {lag}: side stream, eager")
    dec.set_lag(lag, side)
    got = _run(dec)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    dec.prefill()
    torch.cuda.synchronize()
    g = capture(dec.decode)
    replays = {"one graph with a side branch": g.replay,
               "linear graphs joined by events": dec.split_graphs()}
    for name, replay in replays.items():
        say(f"async clustering lag {lag}: side stream, {name}")
        for rep in range(3):
            replay()
            torch.cuda.synchronize()
            for a, b in zip(ref, dec.snapshot()):
                assert torch.equal(a, b), (name, rep)
            torch.ones(1024, device=DEV).cumsum(0)       # eager work between replays
            torch.cuda.synchronize()
    del g, replays

    # oracle: selection at every step, attention around every fork and join
    cent, asg, off, tok, idx, nsel, O = ref
    mu, off_n, tok_n = host_f64(cent), off.cpu().numpy(), tok.cpu().numpy()
    idx_n, nsel_n = idx.cpu().numpy(), nsel.cpu().numpy()
    Kf, Vf = host_f64(layer.K), host_f64(layer.V)
    Qf = host_f64(layer.Q)
    check_attn = set()
    for k in range(T // m):
        for t in (m * (k + 1) - 1, m * (k + 1), m * (k + 1) + lag - 1, m * (k + 1) + lag):
            if 0 <= t < T:
                check_attn.add(t)
    worst = 0.0
    for t in range(T):
        C, pb, npend = dec.schedule[t]
        o_idx, o_ns, _ = oracle.select(Qf[t], mu, off_n, tok_n, C, wl.n_sink, wl.B, G=wl.G,
                                       pending_begin=pb, n_pending=npend)
        assert np.array_equal(nsel_n[t], o_ns), t
        assert np.array_equal(idx_n[t], o_idx), t
        if t in check_attn:
            err = rel_err(host_f64(O[t]), oracle.attn(Qf[t], Kf, Vf, o_idx, o_ns, G=wl.G))
            worst = max(worst, err)
            assert err <= 2e-3, t
    say(f"  lag {lag}: selection exact at {T} steps, attention rel err <= {worst:.2e} at "
        f"{len(check_attn)} steps")


def test_prompt_clustering_overlapped_with_other_work(layer):
    """The prompt's K-means forked onto the side stream while the current
    stream runs other work (standing in for the rest of the layer's
    prefill): the decode that follows equals the run with everything on one
    stream, bit for bit."""
    dec = layer.dec
    say("async clustering: prompt clustering on the side stream")
    dec.set_lag(0, None)
    ref = _run(dec)
    side = torch.cuda.Stream(device=DEV)
    dec.set_lag(0, side)
    a = torch.randn(2048, 2048, device=DEV)
    dec.prefill(overlap=True)
    for _ in range(4):                                    # the caller's own prefill work
        a = a @ a
        a = a / a.abs().max()
    dec.decode()
    torch.cuda.synchronize()
    for x, y in zip(ref, dec.snapshot()):
        assert torch.equal(x, y)
