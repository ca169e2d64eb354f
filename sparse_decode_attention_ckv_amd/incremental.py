"""Decode-time clustering of new tokens, overlapped with decoding.

"ClusterKV: Manipulating LLM KV Cache in Semantic Space for Recallable
Compression", section 语义空间中的聚类 (the tokens generated during decoding
are clustered every m = 320 steps into C+ = 4 new clusters) and section
语义聚类优化 (clustering is started asynchronously and overlapped with the
computation that follows, Fig. 6).

`IncrementalDecoder` runs one layer's decode loop with those increments:
every call is an entry point of libckv (the prompt's and each window's
K-means through ckv_cluster with c_base / t_base / token_base, each step's
selection and attention through ckv_select_attn); this module only orders
the launches on two streams. Decode step t (from 0) attends row L + t, which
the caller has written into K and V before the step. Increment k clusters
rows L + m k .. L + m (k + 1) - 1, the window step m (k + 1) - 1 completes.
With lag D its clusters are first used at step m (k + 1) + D; until then
those rows stay "pending", selected like the sinks (at most m + D pending
rows, so n_sink + m + D <= B). On a side stream the increment is forked
after the step that completes its window and joined before the first step
that uses its clusters, so it overlaps the D steps between.

The two streams touch disjoint memory: an increment writes centroid slots,
CSR offsets and token slots past those the decode steps read (the one shared
word, the offset that ends the last older cluster, is rewritten with the
value it already holds) and reads K rows no step writes after the fork.
Without a side stream the increment runs on the decode stream at the fork
point, which gives the same results.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Tuple

import torch

from . import (CKV_BF16, CKV_F32, AttnDesc, ClusterDesc, SelectDesc, ckv_attn_workspace,
               ckv_cluster, ckv_cluster_workspace_device, ckv_select, ckv_select_attn,
               ckv_select_attn_workspace, ckv_select_workspace, ckv_sparse_attn)

__all__ = ["decode_schedule", "IncrementalDecoder", "capture"]


def decode_schedule(C: int, L: int, m: int, c_plus: int, n_sink: int, B: int, steps: int,
                    lag: int = 0) -> List[Tuple[int, int, int]]:
    """Per decode step t of `steps`: (clusters in use, first pending row,
    pending count). m = 0 means no decode-time clustering: every step uses
    the C prompt clusters and has no pending row. Increment k clusters rows
    L + m k .. L + m (k + 1) - 1, which step m (k + 1) - 1 completes; its
    clusters are used from step m (k + 1) + lag on, and until then the rows
    from the first unclustered one up to the step's own row are pending.
    Raises ValueError for a lag outside 0 .. m - 1 or one whose pending rows
    would not fit the budget."""
    if m == 0:
        if lag != 0:
            raise ValueError("a clustering lag needs decode-time clustering (m > 0)")
        return [(C, 0, 0)] * steps
    if not 0 <= lag < m:
        raise ValueError(f"lag {lag} must be in 0 .. {m - 1} (the clustering period)")
    if n_sink + m + lag > B:
        raise ValueError(f"lag {lag}: n_sink + m + lag = {n_sink + m + lag} exceeds B = {B}")
    sched = []
    for t in range(steps):
        ev = (t - lag) // m if t >= lag else 0
        sched.append((C + c_plus * ev, L + m * ev, t + 1 - m * ev))
    return sched


def capture(fn: Callable[[], None]) -> torch.cuda.CUDAGraph:
    """fn's launches captured as one HIP graph."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


class IncrementalDecoder:
    """One layer's prompt clustering and decode loop with decode-time
    clustering (see the module docstring).

    K, V: the layer's cache, device tensors [H][rows][d] (same strides).
    With decode-time clustering (m > 0) rows >= L + steps and rows
    L .. L + steps - 1 are written by the caller (`before_step(t)` is called
    before step t and may do it); with m = 0 the steps select among the L
    prompt rows only. Q: the steps'
    queries [steps][H*G][d]; results go to idx [steps][H][B], n_sel
    [steps][H] and out [steps][H*G][d] (allocated here unless given).
    `side`: the stream the increments run on (None: the decode stream).
    `fused`: each step as ckv_select_attn, else ckv_select + ckv_sparse_attn
    (the same bits)."""

    def __init__(self, K: torch.Tensor, V: torch.Tensor, Q: torch.Tensor, *, L: int,
                 n_sink: int, C: int, iters: int, B: int, m: int = 320, c_plus: int = 4,
                 lag: int = 0, side: Optional[torch.cuda.Stream] = None, fused: bool = True,
                 before_step: Optional[Callable[[int], None]] = None,
                 idx: Optional[torch.Tensor] = None, n_sel: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None):
        H, rows, d = K.shape
        steps = Q.shape[0]
        need = L + steps if m else L          # decode-time clustering appends a row per step
        if rows < need:
            raise ValueError(f"K has {rows} rows, the decode needs {need}")
        self.K, self.V, self.Q = K, V, Q
        self.L, self.n_sink, self.C, self.iters, self.B = L, n_sink, C, iters, B
        self.m, self.c_plus, self.steps, self.fused = m, c_plus, steps, fused
        self.before_step = before_step
        self.n_ev = steps // m if m else 0
        self.G = Q.shape[1] // H
        dev, dt = K.device, (CKV_BF16 if K.dtype == torch.bfloat16 else CKV_F32)
        c_cap = C + c_plus * self.n_ev
        t_cap = (L - n_sink) + m * self.n_ev
        i32 = dict(dtype=torch.int32, device=dev)
        self.cent = torch.zeros((H, c_cap, d), dtype=torch.float32, device=dev)
        self.asg = torch.empty((H, L), **i32)
        self.off = torch.zeros((H, c_cap + 1), **i32)
        self.tok = torch.zeros((H, t_cap), **i32)
        self.idx = torch.empty((steps, H, B), **i32) if idx is None else idx
        self.nsel = torch.empty((steps, H), **i32) if n_sel is None else n_sel
        self.out = (torch.empty((steps, H * self.G, d), dtype=torch.float32, device=dev)
                    if out is None else out)
        hs = K.stride(0)
        cd = ClusterDesc(H=H, d=d, L=L, k_head_stride=hs, token_base=0, n_sink=n_sink, C=C,
                         iters=iters, dtype=dt, c_base=0, c_cap=c_cap, t_base=0, t_cap=t_cap)
        sd = SelectDesc(H=H, G=self.G, d=d, C=c_cap, c_cap=c_cap, n_sink=n_sink, t_cap=t_cap,
                        pending_begin=0, n_pending=0, B=B, dtype=dt)
        ad = AttnDesc(H=H, G=self.G, d=d, B=B, kv_head_stride=hs, kv_rows=rows, scale=0.0,
                      dtype=dt)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.ws_c = torch.empty(max(ckv_cluster_workspace_device(cd), 1), **u8)
        self.ws_s = torch.empty(max(ckv_select_workspace(sd), 1), **u8)
        self.ws_a = torch.empty(max(ckv_attn_workspace(ad), 1), **u8)
        self.ws_f = torch.empty(max(ckv_select_attn_workspace(sd, ad), 1), **u8)
        if self.n_ev:
            wd = ClusterDesc(H=H, d=d, L=m, k_head_stride=hs, token_base=L, n_sink=0, C=c_plus,
                             iters=iters, dtype=dt, c_base=C, c_cap=c_cap, t_base=L - n_sink,
                             t_cap=t_cap)
            self.ws_w = torch.empty(max(ckv_cluster_workspace_device(wd), 1), **u8)
            self.asg_w = torch.empty((H, m), **i32)
        self.set_lag(lag, side)

    def set_lag(self, lag: int, side: Optional[torch.cuda.Stream]):
        """Steps between an increment's fork and the first step that uses
        it, and the stream it runs on."""
        if lag and not self.n_ev:
            raise ValueError("a lag needs decode-time increments")
        self.lag, self.side = lag, side
        self._prefill_forked = False
        self.schedule = decode_schedule(self.C, self.L, self.m, self.c_plus, self.n_sink, self.B,
                                        self.steps, lag)

    # -- the calls ------------------------------------------------------------
    def prefill(self, overlap: bool = False):
        """K-means of the prompt rows 0 .. L-1 into the first C clusters, on
        the current stream; with overlap (and a side stream), forked onto the
        side stream instead, so the caller's own work on the current stream
        (the rest of the layer's prefill) runs meanwhile, as the page starts
        clustering as soon as the keys exist; decode() joins it before the
        first step."""
        if overlap and self.side is not None:
            self.side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(self.side):
                self._prefill()
            self._prefill_forked = True
        else:
            self._prefill()

    def _prefill(self):
        ckv_cluster(self.K[:, :self.L], self.n_sink, self.C, self.iters, centroids=self.cent,
                    assign=self.asg, csr_offsets=self.off, csr_tokens=self.tok,
                    workspace=self.ws_c)

    def increment(self, k: int):
        """K-means of window k (rows L + m k ..) into c_plus appended clusters,
        on the current stream."""
        m, base = self.m, self.L + self.m * k
        ckv_cluster(self.K[:, base:base + m], 0, self.c_plus, self.iters, token_base=base,
                    centroids=self.cent, assign=self.asg_w, csr_offsets=self.off,
                    csr_tokens=self.tok, c_base=self.C + self.c_plus * k,
                    t_base=base - self.n_sink, workspace=self.ws_w)

    def step(self, t: int):
        """Decode step t: selection with the schedule's clusters and pending
        rows, then attention over the selected rows."""
        C, pb, npend = self.schedule[t]
        if self.fused:
            ckv_select_attn(self.Q[t], self.cent, self.off, self.tok, C, self.B, self.K, self.V,
                            n_sink=self.n_sink, pending_begin=pb, n_pending=npend,
                            idx=self.idx[t], n_sel=self.nsel[t], out=self.out[t],
                            workspace=self.ws_f)
        else:
            ckv_select(self.Q[t], self.cent, self.off, self.tok, C, self.B, n_sink=self.n_sink,
                       pending_begin=pb, n_pending=npend, idx=self.idx[t], n_sel=self.nsel[t],
                       workspace=self.ws_s)
            ckv_sparse_attn(self.Q[t], self.K, self.V, self.idx[t], self.nsel[t],
                            out=self.out[t], workspace=self.ws_a)

    def run_steps(self, a: int, b: int):
        """Steps a .. b - 1 on the current stream, without increments."""
        for t in range(a, b):
            if self.before_step is not None:
                self.before_step(t)
            self.step(t)

    # -- the loop -------------------------------------------------------------
    def decode(self):
        """Every step, eagerly (or under capture), with the increments forked
        onto the side stream and joined `lag` steps later."""
        main, join_t = torch.cuda.current_stream(), None
        if self._prefill_forked:
            main.wait_stream(self.side)
            self._prefill_forked = False
        for t in range(self.steps):
            if t == join_t:
                main.wait_stream(self.side)
                join_t = None
            self.run_steps(t, t + 1)
            if self.n_ev and (t + 1) % self.m == 0 and (t + 1) // self.m <= self.n_ev:
                k = (t + 1) // self.m - 1
                if self.side is None:
                    self.increment(k)
                else:
                    self.side.wait_stream(main)
                    with torch.cuda.stream(self.side):
                        self.increment(k)
                    join_t = t + 1 + self.lag
        if join_t is not None:
            main.wait_stream(self.side)

    def split_graphs(self) -> Callable[[], None]:
        """The decode loop as linear HIP graphs: the steps cut at every fork
        and join point, one graph per piece, one graph per increment. Returns
        a function that replays them on the current stream, forks each
        increment onto the side stream (or runs it in line without one) and
        joins it through an event before the first step that uses it.

        Forks are paced from the host: the steps after a fork point are
        submitted first, then the host waits for the decode stream to reach
        the fork point and only then submits the increment, whose wait is by
        then satisfied. While a side queue holds a wait that is not yet
        satisfied, every launch of the decode chain is slower (measured: about
        4.5 us per step), and so is one graph with the side branch inside."""
        T, D, m = self.steps, self.lag, self.m
        fork = {m * (k + 1): k for k in range(self.n_ev)}          # after step index b - 1
        join = {m * (k + 1) + D: k for k in range(self.n_ev)}      # before step index a
        cuts = sorted({0, T} | {c for c in list(fork) + list(join) if 0 < c < T})
        pieces = [(a, b, capture(lambda a=a, b=b: self.run_steps(a, b)))
                  for a, b in zip(cuts, cuts[1:])]
        incs = [capture(lambda k=k: self.increment(k)) for k in range(self.n_ev)]
        if self.side is None:
            def replay_inline():
                for a, b, g in pieces:
                    g.replay()
                    if b in fork:
                        incs[fork[b]].replay()
            return replay_inline
        forked = [torch.cuda.Event() for _ in range(self.n_ev)]
        done = [torch.cuda.Event() for _ in range(self.n_ev)]
        side = self.side

        def submit(k):
            forked[k].synchronize()
            side.wait_event(forked[k])
            with torch.cuda.stream(side):
                incs[k].replay()
            done[k].record(side)

        def replay():
            main, due, open_ = torch.cuda.current_stream(), None, []
            for a, b, g in pieces:
                if a in join:
                    k = join[a]
                    if due == k:                    # no step between fork and join
                        submit(k)
                        due = None
                    main.wait_event(done[k])
                    open_.remove(k)
                g.replay()
                if due is not None:                 # the steps after the fork are queued
                    submit(due)
                    due = None
                if b in fork:
                    due = fork[b]
                    forked[due].record(main)
                    open_.append(due)
            if due is not None:
                submit(due)
            for k in open_:
                main.wait_event(done[k])
        return replay

    def snapshot(self) -> List[torch.Tensor]:
        """Copies of the clustering state and every step's results."""
        return [x.clone() for x in (self.cent, self.asg, self.off, self.tok, self.idx,
                                    self.nsel, self.out)]
