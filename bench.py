#!/usr/bin/env python3
"""Benchmark of cluster-granular KV selection on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input
(the Llama-3.1-8B-shaped 32k layer by default): ckv_cluster over the prompt
(cosine K-means, 10 iterations) followed by the workload's decode steps,
each one ckv_select_attn call with a fresh query (--separate: ckv_select then
ckv_sparse_attn, bitwise the same). Inputs are resident
in HBM before timing starts. The clustering call and the decode loop are
each captured once as a HIP graph and replayed; every replay's results are
checked bitwise against an eager run before timing.

Prints one JSON line. `value` is the decode-step latency (select + sparse
attention, microseconds per step); the clustering time per layer (with its
p50/p99 over warm replays), the whole-step time and the cold decode step
(the MALL and L2 flushed by a 512 MiB stream before every step) are reported
beside it, and the roofline fractions against both the vendor peaks and the
peaks this GPU achieves on a plain copy and a library GEMM.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("ms per layer ckv_cluster at L=32k; µs/decode step select+sparse attn; "
          "% roofline")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP32_VECTOR_PEAK_TFLOPS = 157.3   # MI355X fp32 vector (256 CUs, 2.4 GHz), TFLOP/s


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3, help="timed steps")
    ap.add_argument("--warmup", type=int, default=1, help="untimed steps")
    ap.add_argument("--workload", default="llama8b_layer_32k")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="decode steps per step (default: the workload's)")
    ap.add_argument("--reps", type=int, default=256,
                    help="back-to-back launches per live per-call timing")
    ap.add_argument("--cluster-reps", type=int, default=20,
                    help="warm clustering replays timed one by one (mean, p50, p99)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure the headline workload only (by default the 32k layer's run "
                         "also reports the other four workloads under \"configs\")")
    ap.add_argument("--separate", action="store_true",
                    help="decode with ckv_select + ckv_sparse_attn instead of ckv_select_attn")
    ap.add_argument("--async-cluster", type=int, default=None, metavar="D",
                    help="incremental workload: run each decode-time clustering on a second "
                         "stream, overlapping the next D decode steps, whose selection keeps "
                         "the window's rows pending until the new clusters are in")
    ap.add_argument("--kv-host", choices=("direct", "cache"), default=None,
                    help="K/V in pinned host memory: attention reads the selected rows from "
                         "there (direct) or through the cluster-granular cache of the rows "
                         "selected in the last R steps (cache)")
    ap.add_argument("--cache-steps", type=int, default=1, metavar="R",
                    help="steps a selected row stays cached (--kv-host cache)")
    ap.add_argument("--query-rho", type=float, default=None,
                    help="step-to-step correlation of an AR(1) query stream (default: "
                         "independent queries; 0.9 with --kv-host)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB ten times and "
                         "exit: the kernel of known traffic that scales the HBM byte counters")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Case:
    """Device-resident inputs and preallocated outputs/workspaces of one
    workload. The prompt's clustering, the decode steps and, for the
    incremental workload, the decode-time increments (forked onto `side`
    and joined `lag` steps later) run through the package's
    IncrementalDecoder; decode step t first appends row L + t of K and V.
    The host-resident K/V variants (`kv_host`) run their own steps."""

    def __init__(self, wl, T, dev, fused=True, lag=0, side=None, kv_host=None, cache_R=1,
                 rho=None):
        import numpy as np
        import torch

        import sparse_decode_attention_ckv_amd as ck
        import synth
        self.wl, self.T, self.fused = wl, T, fused
        t0 = time.time()
        H, G, L, d, C, B = wl.H, wl.G, wl.L, wl.d, wl.C, wl.B
        self.inc = wl.append_steps > 0
        self.n_ev = T // wl.m_every if self.inc else 0
        Lcap = L + T if self.inc else L
        K, V, _ = synth.make_kv(wl, L=L, L_cap=Lcap)
        if rho is None:
            Q, _ = synth.make_query_steps(wl, T)
        else:
            Q, _ = synth.make_query_stream(wl, T, rho)

        def bf(a):
            if wl.dtype == "bf16":
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                    torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
        # K and V as the two halves of one cache tensor (same strides), so an
        # appended row of both is one copy
        self.KV = bf(np.stack([K, V]))
        self.K, self.V, self.Q = self.KV[0], self.KV[1], bf(Q)
        if self.inc:
            app = [synth.make_appended(wl, h, T) for h in range(H)]
            self.KVa = bf(np.stack([np.stack([x[0] for x in app]), np.stack([x[1] for x in app])]))
        log(f"inputs drawn in {time.time() - t0:.1f}s")
        from sparse_decode_attention_ckv_amd.incremental import IncrementalDecoder
        # the prompt's clustering, the decode steps and (incremental workload)
        # the decode-time increments on their own stream: the package's helper
        self.dec = IncrementalDecoder(
            self.K, self.V, self.Q, L=L, n_sink=wl.n_sink, C=C, iters=wl.iters, B=B,
            m=wl.m_every if self.inc else 0, c_plus=wl.c_plus, fused=fused,
            before_step=self.append if self.inc else None)
        d_ = self.dec
        self.cent, self.asg, self.off, self.tok = d_.cent, d_.asg, d_.off, d_.tok
        self.idx, self.nsel, self.O = d_.idx, d_.nsel, d_.out
        self.ws_c, self.ws_s, self.ws_a, self.ws_f = d_.ws_c, d_.ws_s, d_.ws_a, d_.ws_f
        u8 = dict(dtype=torch.uint8, device=dev)
        self.ck = ck
        self.set_lag(lag, side)
        # K/V in pinned host memory: attention reads the selected rows from
        # there directly, or through the cluster-granular cache
        self.kv_host = kv_host
        if kv_host is not None:
            assert not self.inc, "host-resident K/V is measured on the prompt workloads"
            self.Kh = torch.empty(self.K.shape, dtype=self.K.dtype, pin_memory=True)
            self.Vh = torch.empty(self.V.shape, dtype=self.V.dtype, pin_memory=True)
            self.Kh.copy_(self.K.cpu())
            self.Vh.copy_(self.V.cpu())
            self.stats_acc = torch.zeros((H, 5), dtype=torch.int64, device=dev)
            self.count_stats = False      # summing the statistics is bookkeeping: eager only
            if kv_host == "cache":
                self.cdesc = ck.cache_desc(self.Kh, self.asg, self.off, self.tok, C, B, cache_R,
                                           n_sink=wl.n_sink)
                self.cst = ck.cache_state(self.cdesc, dev)
                ad_c = ck.AttnDesc(H=H, G=G, d=d, B=B, kv_head_stride=self.cst["rows"] * d,
                                   kv_rows=self.cst["rows"], scale=0.0, dtype=ck.CKV_BF16)
                self.ws_ac = torch.empty(ck.ckv_attn_workspace(ad_c), **u8)

    def set_lag(self, lag, side):
        self.dec.set_lag(lag, side)
        self.lag, self.side, self.sched = lag, side, self.dec.schedule

    def cluster(self):
        self.dec.prefill()

    def append(self, t):
        self.KV[:, :, self.wl.L + t].copy_(self.KVa[:, :, t])

    def increment(self, k):
        self.dec.increment(k)

    def select(self, t):
        wl = self.wl
        C, pb, npend = self.sched[t]
        self.ck.ckv_select(self.Q[t], self.cent, self.off, self.tok, C, wl.B,
                           n_sink=wl.n_sink, pending_begin=pb, n_pending=npend,
                           idx=self.idx[t], n_sel=self.nsel[t], workspace=self.ws_s)

    def attn(self, t):
        self.ck.ckv_sparse_attn(self.Q[t], self.K, self.V, self.idx[t], self.nsel[t],
                                out=self.O[t], workspace=self.ws_a)

    def select_attn(self, t):
        wl = self.wl
        C, pb, npend = self.sched[t]
        self.ck.ckv_select_attn(self.Q[t], self.cent, self.off, self.tok, C, wl.B, self.K, self.V,
                                n_sink=wl.n_sink, pending_begin=pb, n_pending=npend,
                                idx=self.idx[t], n_sel=self.nsel[t], out=self.O[t],
                                workspace=self.ws_f)

    def host_step(self, t):
        """Selection, then attention over host-resident K/V: read directly,
        or through the cache of the rows selected in the last R steps."""
        self.select(t)
        if self.kv_host == "direct":
            self.ck.ckv_sparse_attn(self.Q[t], self.Kh, self.Vh, self.idx[t], self.nsel[t],
                                    out=self.O[t], workspace=self.ws_a)
            return
        st = self.cst
        cK, cV = self.ck.ckv_cache_step(self.cdesc, t, self.idx[t], self.nsel[t], self.asg,
                                        self.off, self.tok, self.Kh, self.Vh, st)
        self.ck.ckv_sparse_attn(self.Q[t], cK, cV, st["idx_cache"], self.nsel[t],
                                kv_rows=st["rows"], out=self.O[t], workspace=self.ws_ac)
        if self.count_stats:
            self.stats_acc.add_(st["stats"])

    def steps(self, a, b):
        """Decode steps a .. b - 1 (0-based), without increments."""
        if self.kv_host is not None:
            if a == 0:
                if self.count_stats:
                    self.stats_acc.zero_()
                if self.kv_host == "cache":
                    self.cst["ring"].zero_()
            for t in range(a, b):
                self.host_step(t)
            return
        self.dec.run_steps(a, b)

    def decode(self):
        if self.kv_host is not None:
            self.steps(0, self.T)
            return
        self.dec.decode()

    def split_graphs(self):
        """The decode loop as linear graphs with side-stream increments (the
        package's IncrementalDecoder.split_graphs)."""
        return self.dec.split_graphs()

    def snapshot(self):
        extra = [] if self.kv_host is None else [self.stats_acc]
        return [x.clone() for x in (self.cent, self.asg, self.off, self.tok, self.idx,
                                    self.nsel, self.O, *extra)]


from sparse_decode_attention_ckv_amd.incremental import capture  # noqa: E402


def time_graph(g, reps=1):
    """Average ms of `reps` back-to-back replays, HIP events on the stream the
    graph is launched on (the current stream)."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def pct(xs, p):
    """p-th percentile of the sorted list xs (nearest rank)."""
    k = max(0, min(len(xs) - 1, -(-len(xs) * p // 100) - 1))
    return xs[k]


def measured_peaks(dev):
    """What this GPU achieves on plain work, beside the vendor figures: HBM
    bandwidth of a 1 GiB device-to-device copy (bytes read + written per
    second) and bf16 matrix throughput of an 8192^3 GEMM (hipBLASLt through
    torch.mm, contiguous operands), each the best of 5 timed runs."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    M = 8192
    a = torch.randn((M, M), device=dev).to(torch.bfloat16)
    b = torch.randn((M, M), device=dev).to(torch.bfloat16)
    dst.copy_(src)
    c = torch.mm(a, b)
    torch.cuda.synchronize()

    def best(fn):
        t = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e-3)
        return min(t)
    copy_s = best(lambda: dst.copy_(src))
    gemm_s = best(lambda: torch.mm(a, b, out=c))
    del src, dst, a, b, c
    return {"hbm_copy_GB/s": round(2 * n / copy_s / 1e9, 1),
            "bf16_gemm_TFLOP/s": round(2 * M ** 3 / gemm_s / 1e12, 1),
            "method": "1 GiB device copy; 8192^3 bf16 torch.mm; best of 5 each"}


def copy_calibration(mib):
    """Ten copies of `mib` MiB between two device buffers: each reads and
    writes exactly mib * 2^20 bytes, so the byte counters of its kernel give
    the scale of the counters for any other kernel."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert bool(dst.eq(1).all())
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 10}), flush=True)


# HBM traffic of the dominant kernel, from the byte counters of a profiled run
# (FETCH_SIZE and WRITE_SIZE, scaled by the copy calibration). The record
# holds the hash of the kernel's sources at the time; once they change the
# figure no longer applies and is reported as null.
KERNEL_SOURCES = {
    "ckv_select": ["select.hip", "sel_dev.h", "ckv_dev.h"],
    "ckv_sparse_attn": ["attn.hip", "attn_dev.h", "ckv_dev.h"],
    "ckv_select_attn": ["decode.hip", "select.hip", "sel_dev.h", "attn.hip", "attn_dev.h",
                        "ckv_dev.h"],
    "ckv_cluster": ["cluster.hip", "cluster_dev.h", "ckv_dev.h"],
}


def sources_sha256(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sparse_decode_attention_ckv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            line = line.strip().strip("`")
            if ":" in line and line.split(":")[0] in ("source_sha256", "bytes_per_launch"):
                k, v = line.split(":", 1)
                rec[k] = v.strip()
    if rec.get("source_sha256") != sources_sha256(kernel) or "bytes_per_launch" not in rec:
        return None
    return int(float(rec["bytes_per_launch"]))


def host_cpu():
    """The host's CPU model (/proc/cpuinfo) and its logical CPU count."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def cpu_baseline(case, sample_steps, cluster_heads, threads, cluster_tokens=None,
                 full_cluster=False, increment=False):
    """The oracle as it stands on a bounded sample of the same workload.

    Decode: `sample_steps` steps (all KV heads, each step's selection on the
    GPU's centroids and CSR with that step's cluster count and pending rows,
    then attention), timed on one core. Clustering: with `full_cluster` the
    whole K-means of the layer (every iteration, every head), measured;
    otherwise one K-means iteration on `cluster_heads` heads -- on their first
    `cluster_tokens` rows when given, which scales linearly with the rows --
    extrapolated to the layer and labelled so. With `increment`, one
    decode-time clustering event (the newest window into c_plus clusters,
    all iterations, all heads) is timed as well. With threads > 1 the decode
    sample and the clustering sample also run as independent per-head oracle
    instances on that many host threads (the oracle stays single-threaded;
    its C calls release the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    wl = case.wl
    G = wl.G
    sample_steps = max(1, min(sample_steps, case.T))
    cluster_heads = max(1, min(cluster_heads, wl.H))
    mu = case.cent.double().cpu().numpy()
    off = case.off.cpu().numpy()
    tok = case.tok.cpu().numpy()
    Kf = case.K.double().cpu().numpy()
    Vf = case.V.double().cpu().numpy()
    Qf = case.Q[:sample_steps].double().cpu().numpy()
    sched = case.sched
    oracle.select(Qf[0], mu, off, tok, wl.C, wl.n_sink, wl.B, G=G)   # load the library

    def step(t, h0=0, h1=None):
        h1 = wl.H if h1 is None else h1
        C, pb, npend = sched[t]
        q = Qf[t, h0 * G:h1 * G]
        idx, ns, _ = oracle.select(q, mu[h0:h1], off[h0:h1], tok[h0:h1], C, wl.n_sink, wl.B,
                                   G=G, pending_begin=pb, n_pending=npend)
        oracle.attn(q, Kf[h0:h1], Vf[h0:h1], idx, ns, G=G)

    Lc = wl.L if cluster_tokens is None else min(wl.L, wl.n_sink + cluster_tokens)

    def iterate_head(h):
        K = Kf[h, :Lc]
        mu0 = oracle.init_centroids(Kf[h, :wl.L], wl.n_sink, wl.C)
        a, _ = oracle.assign(K, wl.n_sink, mu0, mode=oracle.MIRROR)
        oracle.update(K, wl.n_sink, a, mu0, mode=oracle.MIRROR)

    def timed(fn, items, n):
        t0 = time.perf_counter()
        if n == 1:
            for x in items:
                fn(x)
        else:
            with ThreadPoolExecutor(max_workers=n) as ex:
                list(ex.map(fn, items))
        return time.perf_counter() - t0

    t0 = time.perf_counter()
    for t in range(sample_steps):
        step(t)
    dec_s = (time.perf_counter() - t0) / sample_steps
    Lp = wl.L - wl.n_sink
    out = {"value": round(dec_s * 1e6, 1), "unit": "us/decode_step", "cores": 1,
           "kind": "oracle"}
    if full_cluster:
        t0 = time.perf_counter()
        oracle.cluster(Kf[:, :wl.L], wl.n_sink, wl.C, wl.iters, mode=oracle.EXACT
                       if wl.dtype != "bf16" else oracle.MIRROR)
        out["cluster_ms_per_layer"] = round((time.perf_counter() - t0) * 1e3, 2)
        clus = f"the whole K-means of the layer ({wl.iters} iterations, {wl.H} heads), measured"
    else:
        it_s = timed(iterate_head, range(cluster_heads), 1) / cluster_heads
        scale = Lp / (Lc - wl.n_sink)
        out["cluster_ms_per_layer_extrapolated"] = round(it_s * scale * wl.H * wl.iters * 1e3, 1)
        clus = (f"1 K-means iteration on {cluster_heads} of {wl.H} heads"
                + (f" over their first {Lc - wl.n_sink} of {Lp} rows" if Lc < wl.L else "")
                + f", extrapolated to {wl.H} heads x {wl.iters} iterations"
                + (" x the rows" if Lc < wl.L else ""))
    if increment:
        m = wl.m_every
        t0 = time.perf_counter()
        oracle.cluster(Kf[:, wl.L:wl.L + m], 0, wl.c_plus, wl.iters, mode=oracle.MIRROR,
                       token_base=wl.L)
        out["increment_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
        clus += f"; one decode-time increment ({m} rows into {wl.c_plus} clusters, all heads)"
    out["sample"] = (f"{sample_steps} decode steps (select + sparse attention, all {wl.H} KV "
                     f"heads) and {clus}; C oracle (fp64), single-threaded")
    n = max(1, min(threads, wl.H))
    if n > 1:
        dec_n = timed(lambda h: [step(t, h, h + 1) for t in range(sample_steps)],
                      range(wl.H), n) / sample_steps
        it_n = timed(iterate_head, range(cluster_heads), n) * wl.H / cluster_heads
        out["per_head_threads"] = {
            "cores": n, "value": round(dec_n * 1e6, 1), "unit": "us/decode_step",
            "cluster_ms_per_layer_extrapolated": round(
                it_n * (Lp / (Lc - wl.n_sink)) * wl.iters * 1e3, 1),
            "sample": f"the same sample as independent per-head oracle calls on {n} threads"}
    out["host_cpu"] = host_cpu()
    out["host_threads"] = os.cpu_count()
    return out


def run_workload(name, args, peaks, *, steps, warmup, reps, cluster_reps, decode_steps=None,
                 async_cluster=None, kv_host_mode=None, cpu_sample=None):
    """Everything measured on one workload: the whole step (clustering +
    decode loop) replayed from HIP graphs checked bitwise against an eager
    run, clustering latency over warm replays, cold decode steps, live
    per-call timings and their rooflines, and the oracle on a bounded
    sample. Returns the workload's record."""
    import torch

    import synth
    dev = "cuda:0"
    wl = synth.workload(name)
    T = wl.steps if decode_steps is None else decode_steps
    lag, side = 0, None
    if async_cluster is not None:
        lag, side = async_cluster, torch.cuda.Stream(device=dev)
    rho = args.query_rho
    if kv_host_mode is not None and rho is None:
        rho = 0.9
    case = Case(wl, T, dev, fused=not args.separate, lag=lag, side=side, kv_host=kv_host_mode,
                cache_R=args.cache_steps, rho=rho)

    # eager reference run
    case.cluster()
    if case.kv_host is not None:
        case.count_stats = True
    case.decode()
    torch.cuda.synchronize()
    ref = case.snapshot()
    if case.kv_host is not None:
        case.count_stats = False
    kv_host = None
    if case.kv_host is not None:
        # the same queries on the device-resident path give the same outputs
        mode, case.kv_host = case.kv_host, None
        case.decode()
        torch.cuda.synchronize()
        assert torch.equal(case.O, ref[6]) and torch.equal(case.idx, ref[4]), \
            "host-resident decode differs from the device-resident one"
        case.kv_host = mode
        log(f"host-resident ({mode}) decode matches the device-resident decode bitwise")
        acc = ref[7].cpu()
        n_sel_rows = int(ref[5].cpu().to(torch.int64).sum())
        row_bytes = 2 * wl.d * 2                      # one K row and one V row, bf16
        if mode == "direct":
            host_rows = n_sel_rows
        else:
            host_rows = int(acc[:, 1].sum()) + wl.H * wl.n_sink   # + the sinks, once
        hit = int(acc[:, 0].sum())
        kv_host = {"mode": mode, "query_rho": rho,
                   "host_bytes_per_step": round(host_rows * row_bytes / T),
                   "selected_rows_per_step": round(n_sel_rows / T, 1)}
        if mode == "cache":
            kv_host.update({
                "R": args.cache_steps,
                "cluster_rows_from_cache": round(hit / max(1, hit + int(acc[:, 1].sum())), 4),
                "clusters_whole_in_cache": round(int(acc[:, 2].sum()) /
                                                 max(1, int(acc[:, 3].sum())), 4)})

    # graphs: the clustering call and the whole decode loop (with side-stream
    # increments: linear graphs joined by events)
    g_cluster = capture(case.cluster)
    if side is None:
        g_decode = capture(case.decode)
        decode_replay = g_decode.replay
    else:
        decode_replay = case.split_graphs()
    for rep in range(2):
        g_cluster.replay()
        decode_replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, case.snapshot()):
            assert torch.equal(a, b), "graph replay differs from the eager run"
        torch.cuda.synchronize()
    log("graph replays match the eager run bitwise")

    def step():
        g_cluster.replay()
        decode_replay()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * steps)]
    t_wall = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(steps):
        ev[3 * k].record()
        g_cluster.replay()
        ev[3 * k + 1].record()
        decode_replay()
        ev[3 * k + 2].record()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / steps
    cl_ms = sum(ev[3 * k].elapsed_time(ev[3 * k + 1]) for k in range(steps)) / steps
    dec_ms = sum(ev[3 * k + 1].elapsed_time(ev[3 * k + 2]) for k in range(steps)) / steps
    dec_us = dec_ms * 1e3 / T
    if kv_host is not None:
        kv_host["host_GB/s_over_step"] = round(kv_host["host_bytes_per_step"] / dec_us / 1e3, 2)
        log(f"host-resident {kv_host['mode']}: {kv_host['host_bytes_per_step']} host bytes per "
            f"step ({kv_host['host_GB/s_over_step']} GB/s over the step)"
            + (f", {kv_host['cluster_rows_from_cache']:.3f} of cluster rows from the cache"
               if kv_host["mode"] == "cache" else ""))
    log(f"step {ms_step:.3f} ms (wall {wall / steps * 1e3:.3f} ms): cluster {cl_ms:.3f} ms, "
        f"decode {dec_us:.2f} us/step")

    # clustering latency distribution: warm replays, each between HIP events
    cl_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(cluster_reps)]
    for a, b in cl_ev:
        a.record()
        g_cluster.replay()
        b.record()
    torch.cuda.synchronize()
    cl_reps = sorted(a.elapsed_time(b) for a, b in cl_ev)

    # cold decode steps: a 512 MiB read-modify-write before every step evicts
    # the MALL and the L2, as the other layers of a model would between two
    # steps of one layer; cold step = (T(flush + step) - T(flush)) / n
    flush_buf = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
    n_cold = min(T, 64)
    g_fs = capture(lambda: [(flush_buf.add_(1), case.steps(t, t + 1)) for t in range(n_cold)])
    g_f = capture(lambda: [flush_buf.add_(1) for _ in range(n_cold)])
    cold_us = (time_graph(g_fs, 3) - time_graph(g_f, 3)) * 1e3 / n_cold
    del g_fs, g_f, flush_buf
    log(f"cluster over {len(cl_reps)} warm replays: p50 {pct(cl_reps, 50):.3f} ms, "
        f"p99 {pct(cl_reps, 99):.3f} ms; cold decode step {cold_us:.2f} us")

    # live per-call timings (back-to-back launches of one call, HIP events)
    g_sel = capture(lambda: [case.select(0) for _ in range(reps)])
    g_att = capture(lambda: [case.attn(0) for _ in range(reps)])
    g_fus = capture(lambda: [case.select_attn(0) for _ in range(reps)])
    sel_us = time_graph(g_sel) * 1e3 / reps
    att_us = time_graph(g_att) * 1e3 / reps
    fus_us = time_graph(g_fus) * 1e3 / reps
    inc_ms = None
    if case.inc:                          # one decode-time clustering event, back to back
        g_inc = capture(lambda: [case.increment(0) for _ in range(16)])
        inc_ms = time_graph(g_inc) / 16
    torch.cuda.synchronize()
    H, G, d, C, B = wl.H, wl.G, wl.d, wl.C, wl.B
    n_sel = case.nsel[0].cpu()
    e = 2 if wl.dtype == "bf16" else 4      # element bytes
    att_bytes = sum(2 * int(n) * d * e + 4 * B + G * d * e + G * d * 4 for n in n_sel)
    sel_bytes = sum(C * d * 4 + 4 * (C + 1) + 4 * (int(n) - wl.n_sink) + 4 * B + G * d * e
                    for n in n_sel)
    # the fused step reads q once and never reads idx back
    fus_bytes = sel_bytes + att_bytes - H * (G * d * e + 4 * B)
    Lp = wl.L - wl.n_sink
    assign_flop = 2.0 * Lp * C * d * H * wl.iters
    kernels = {
        "ckv_sparse_attn": {"us_per_call": round(att_us, 3), "bytes": att_bytes,
                            "GB/s": round(att_bytes / att_us / 1e3, 1),
                            "calls_per_step": T},
        "ckv_select": {"us_per_call": round(sel_us, 3), "bytes": sel_bytes,
                       "GB/s": round(sel_bytes / sel_us / 1e3, 1),
                       "calls_per_step": 0 if case.fused else T},
        "ckv_select_attn": {"us_per_call": round(fus_us, 3), "bytes": fus_bytes,
                            "GB/s": round(fus_bytes / fus_us / 1e3, 1),
                            "calls_per_step": T if case.fused else 0},
        "ckv_cluster": {"ms_per_call": round(cl_ms, 4), "assign_flop": assign_flop,
                        "assign_TFLOP/s_over_whole_call": round(assign_flop / cl_ms / 1e9, 1),
                        "calls_per_step": 1},
    }
    if case.fused:
        kernels["ckv_sparse_attn"]["calls_per_step"] = 0
        share = {"ckv_select_attn": fus_us * T / 1e3, "ckv_cluster": cl_ms}
    else:
        share = {"ckv_sparse_attn": att_us * T / 1e3, "ckv_select": sel_us * T / 1e3,
                 "ckv_cluster": cl_ms}
    if case.inc:
        kernels["ckv_cluster_increment"] = {"ms_per_call": round(inc_ms, 4),
                                            "calls_per_step": case.n_ev}
    dom = max(share, key=share.get)
    if dom == "ckv_cluster" and wl.dtype != "bf16":
        # fp32 keys: the assignment's dot products are vector fp32 FMAs
        roof = {"kernel": dom, "bound": "alu", "achieved": round(assign_flop / cl_ms / 1e9, 2),
                "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s"}
    elif dom == "ckv_cluster":
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(assign_flop / cl_ms / 1e9, 2),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        k = kernels[dom]
        roof = {"kernel": dom, "bound": "hbm", "achieved": k["GB/s"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    if roof["bound"] != "alu":
        roof["measured_peak"] = (peaks["bf16_gemm_TFLOP/s"] if roof["bound"] == "mfma"
                                 else peaks["hbm_copy_GB/s"])
        roof["frac_of_measured_peak"] = round(roof["achieved"] / roof["measured_peak"], 4)
    roof["traffic"] = recorded_traffic(dom, wl.name)
    kernels["ckv_cluster"]["assign_frac_of_measured_gemm"] = round(
        assign_flop / cl_ms / 1e9 / peaks["bf16_gemm_TFLOP/s"], 4)
    log(f"measured peaks: HBM copy {peaks['hbm_copy_GB/s']} GB/s, bf16 GEMM "
        f"{peaks['bf16_gemm_TFLOP/s']} TFLOP/s")
    if dom in ("ckv_select_attn", "ckv_sparse_attn", "ckv_select"):
        # the same call with the MALL and L2 flushed before it
        cold_gbs = (fus_bytes if case.fused else sel_bytes + att_bytes) / cold_us / 1e3
        roof["cold"] = {"us_per_call": round(cold_us, 3), "achieved": round(cold_gbs, 1),
                        "frac": round(cold_gbs / HBM_PEAK_GBS, 4),
                        "frac_of_measured_peak": round(cold_gbs / peaks["hbm_copy_GB/s"], 4)}
    log(f"per call: select {sel_us:.2f} us, attn {att_us:.2f} us, select_attn {fus_us:.2f} us"
        + (f", decode-time clustering {inc_ms * 1e3:.1f} us per event" if case.inc else "")
        + f"; dominant {dom}")

    cpu = None
    if cpu_sample is not None:
        log(f"{wl.name}: timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(case, **cpu_sample)

    out = {
        "value": round(dec_us, 3), "ms_per_step": round(ms_step, 4), "wl": wl,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "config": {"workload": wl.name, "kv_heads": H, "q_heads_per_kv": G, "d": d, "L": wl.L,
                   "n_sink": wl.n_sink, "C": C, "iters": wl.iters, "B": B,
                   "decode_steps": T, "parallelism": "none (1 GPU)",
                   **({"append_steps": T, "cluster_every": wl.m_every,
                       "clusters_per_increment": wl.c_plus, "cluster_lag_steps": lag,
                       "cluster_stream": "side" if side is not None else "decode"}
                      if case.inc else {})},
        "cluster_ms_per_layer": round(cl_ms, 4),
        "cluster_ms_warm_reps": {"n": len(cl_reps), "mean": round(sum(cl_reps) / len(cl_reps), 4),
                                 "p50": round(pct(cl_reps, 50), 4),
                                 "p99": round(pct(cl_reps, 99), 4)},
        "decode_us_per_step": round(dec_us, 3),
        "decode_cold_us_per_step": round(cold_us, 3),
        "decode_path": ("ckv_select + ckv_sparse_attn over host K/V" if kv_host_mode == "direct"
                        else "ckv_select + ckv_cache_step + ckv_sparse_attn over the cache"
                        if kv_host_mode == "cache"
                        else "ckv_select + ckv_sparse_attn" if args.separate
                        else "ckv_select_attn"),
        **({"kv_host": kv_host} if kv_host else {}),
        "roofline": roof,
        "measured_peaks": peaks,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    del case
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# The other workloads reported beside the headline one, and the bounded
# oracle sample of each (see cpu_baseline).
OTHER_CONFIGS = {
    "single_head_fp32_2k": dict(sample_steps=1, cluster_heads=1, threads=1, full_cluster=True),
    "llama8b_layer_32k_batch8": dict(sample_steps=4, cluster_heads=2, threads=1),
    "llama8b_layer_32k_incremental": dict(sample_steps=16, cluster_heads=1, threads=1,
                                          increment=True),
    "llama8b_layer_128k": dict(sample_steps=4, cluster_heads=1, threads=1, cluster_tokens=4096),
}


def config_summary(rec):
    """The part of a workload's record reported per config."""
    keys = ("value", "dtype", "config", "cluster_ms_per_layer", "cluster_ms_warm_reps",
            "decode_us_per_step", "decode_cold_us_per_step", "decode_path", "roofline",
            "kernels", "cpu_baseline")
    out = {k: rec[k] for k in keys if k in rec}
    out["unit"] = "us/decode_step"
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): every KV head is an independent problem, so a multi-GPU run would "
              "shard heads with no communication; it is not built or measured here.",
              flush=True)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    peaks = measured_peaks("cuda:0")
    headline_cpu = None if args.no_cpu_baseline else dict(
        sample_steps=128, cluster_heads=8, threads=min(16, os.cpu_count() or 1))
    rec = run_workload(args.workload, args, peaks, steps=args.steps, warmup=args.warmup,
                       reps=args.reps, cluster_reps=args.cluster_reps,
                       decode_steps=args.decode_steps, async_cluster=args.async_cluster,
                       kv_host_mode=args.kv_host, cpu_sample=headline_cpu)
    configs = None
    plain = (args.workload == "llama8b_layer_32k" and args.decode_steps is None
             and args.async_cluster is None and args.kv_host is None and not args.separate)
    if plain and not args.no_configs:
        configs = {}
        for name, sample in OTHER_CONFIGS.items():
            log(f"config {name} ...")
            r = run_workload(name, args, peaks, steps=2, warmup=1, reps=64, cluster_reps=5,
                             cpu_sample=None if args.no_cpu_baseline else sample)
            configs[name] = config_summary(r)
    wl = rec["wl"]
    out = {
        "metric": METRIC, "value": rec["value"], "unit": "us/decode_step",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"], "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": rec["dtype"], "data": "synthetic",
        "config": rec["config"],
        **{k: v for k, v in rec.items() if k not in ("value", "ms_per_step", "wl", "dtype",
                                                       "config")},
    }
    out["measured_peaks"] = peaks
    if configs is not None:
        out["configs"] = configs
    del wl
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
