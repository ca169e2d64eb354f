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

import bench
import oracle
import synth
from tests.gpu_helpers import DEV, host_f64, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def case():
    wl = synth.workload("llama8b_layer_32k_incremental")
    say(f"async clustering: drawing the {wl.name} inputs")
    return bench.Case(wl, wl.append_steps, DEV)


def _run(case):
    case.cluster()
    case.decode()
    torch.cuda.synchronize()
    return case.snapshot()


@pytest.mark.parametrize("lag", [0, 32, 319])
def test_overlapped_increments_match_one_stream(case, lag):
    wl, T, m = case.wl, case.T, case.wl.m_every
    side = torch.cuda.Stream(device=DEV)
    say(f"async clustering lag {lag}: one stream")
    case.set_lag(lag, None)
    ref = _run(case)
    say(f"async clustering lag {lag}: side stream, eager")
    case.set_lag(lag, side)
    got = _run(case)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    case.cluster()
    torch.cuda.synchronize()
    g = bench.capture(case.decode)
    replays = {"one graph with a side branch": g.replay,
               "linear graphs joined by events": case.split_graphs()}
    for name, replay in replays.items():
        say(f"async clustering lag {lag}: side stream, {name}")
        for rep in range(3):
            replay()
            torch.cuda.synchronize()
            for a, b in zip(ref, case.snapshot()):
                assert torch.equal(a, b), (name, rep)
            torch.ones(1024, device=DEV).cumsum(0)       # eager work between replays
            torch.cuda.synchronize()
    del g, replays

    # oracle: selection at every step, attention around every fork and join
    cent, asg, off, tok, idx, nsel, O = ref
    mu, off_n, tok_n = host_f64(cent), off.cpu().numpy(), tok.cpu().numpy()
    idx_n, nsel_n = idx.cpu().numpy(), nsel.cpu().numpy()
    Kf, Vf = host_f64(case.K), host_f64(case.V)
    Qf = host_f64(case.Q)
    check_attn = set()
    for k in range(T // m):
        for t in (m * (k + 1) - 1, m * (k + 1), m * (k + 1) + lag - 1, m * (k + 1) + lag):
            if 0 <= t < T:
                check_attn.add(t)
    worst = 0.0
    for t in range(T):
        C, pb, npend = case.sched[t]
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
