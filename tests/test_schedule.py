"""Host logic of the incremental decode schedule (no GPU).

The schedule gives each decode step the clusters it may use and the range of
rows it must treat as pending. It is checked against a direct simulation of
the events: increment k clusters the m rows that step m (k + 1) completes,
is forked after that step and joined `lag` steps later, and a step may use
only the increments joined before it; every row appended so far that no used
increment covers must be pending, and nothing else.
"""
import pytest

import synth
from sparse_decode_attention_ckv_amd.incremental import decode_schedule

WL = synth.workload("llama8b_layer_32k_incremental")


def _schedule(wl, T, lag=0):
    return decode_schedule(wl.C, wl.L, wl.m_every, wl.c_plus, wl.n_sink, wl.B, T, lag)


def _simulate(wl, T, lag):
    m, out = wl.m_every, []
    joins = [m * (k + 1) + lag for k in range(T // m)]      # first step index that may use k
    for t in range(T):
        used = sum(1 for j in joins if j <= t)
        rows = range(wl.L, wl.L + t + 1)                    # rows appended by steps 0..t
        pending = [r for r in rows if r >= wl.L + m * used]
        out.append((wl.C + wl.c_plus * used, pending))
    return out


@pytest.mark.parametrize("lag", [0, 1, 32, 319])
def test_schedule_matches_event_simulation(lag):
    T = WL.append_steps
    sched = _schedule(WL, T, lag)
    sim = _simulate(WL, T, lag)
    assert len(sched) == T
    for t, ((C, pb, npend), (C_s, pend)) in enumerate(zip(sched, sim)):
        assert C == C_s, t
        assert npend == len(pend) and pb == pend[0] and pb + npend - 1 == WL.L + t, t
        assert WL.n_sink + npend <= WL.B, t
    assert max(s[2] for s in sched) == WL.m_every + lag
    # lag 0 is the schedule of increments used right after they are due
    if lag == 0:
        ev = [t // WL.m_every for t in range(T)]
        assert sched == [(WL.C + WL.c_plus * e, WL.L + WL.m_every * e, t + 1 - WL.m_every * e)
                         for t, e in enumerate(ev)]


@pytest.mark.parametrize("lag", [-1, WL.m_every, WL.B])
def test_schedule_rejects_bad_lag(lag):
    with pytest.raises(ValueError):
        _schedule(WL, WL.append_steps, lag)


def test_schedule_static_workload():
    wl = synth.workload("llama8b_layer_32k")
    assert decode_schedule(wl.C, wl.L, 0, 0, wl.n_sink, wl.B, 4) == [(wl.C, 0, 0)] * 4
    with pytest.raises(ValueError):
        decode_schedule(wl.C, wl.L, 0, 0, wl.n_sink, wl.B, 4, lag=3)
