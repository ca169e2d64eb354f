"""Seeded random-shape parity sweep on the GPU.

The parity tests name their edge cases one by one; this sweep draws mixed
shapes from fixed seeds and holds every path to the same bar:

* decode: KV heads, query heads per KV head, cluster count (up to 2048, so
  both LDS sizes of the cut run), window length, sinks, pending rows, budget
  (below, at and above the window) and dtype. The fused call must be bitwise
  the separate calls, the selection bit-exact against the oracle, and the
  attention within 2e-3 (bf16) or 1e-5 (fp32) of the fp64 attention
  (test_gpu_fused's checks);
* clustering: heads, sinks, cluster count (both CSR versions, C <= 512 and
  above, and the small-window kernel), window length, iterations and dtype,
  with per-iteration parity: labels outside the margin exact, the CSR of the
  GPU's labels exact, centroids within 1e-4 (lloyd_parity).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import lloyd_parity, say, to_dev
from tests.test_gpu_fused import test_fused_equals_separate_and_oracle as fused_case

pytestmark = pytest.mark.gpu


def _decode_cfg(seed):
    r = np.random.default_rng(7100 + seed)
    dtype = "f32" if seed % 8 == 5 else "bf16"
    H = int(r.integers(1, 13))
    G = int(r.integers(1, 9))
    C = int(r.integers(600, 2049)) if seed % 4 == 0 else int(r.integers(1, 600))
    Lp = int(r.integers(C, C + 6000))
    n_sink = int(r.choice([0, 16, int(r.integers(1, 40))]))
    n_pending = int(r.choice([0, 0, int(r.integers(1, 200))]))
    head = n_sink + n_pending
    B = int(r.integers(max(1, head), head + Lp + 300))
    return H, G, C, Lp, B, n_sink, n_pending, dtype


def _cluster_cfg(seed):
    r = np.random.default_rng(7300 + seed)
    dtype = "f32" if seed % 6 == 1 else "bf16"
    H = 1 if dtype == "f32" else int(r.integers(1, 4))
    n_sink = int(r.choice([0, 16, int(r.integers(1, 30))]))
    kind = seed % 3
    if kind == 0:                         # small window: the one-launch kernel (bf16)
        C = int(r.integers(1, 17))
        L = n_sink + int(r.integers(C, 1025))
    elif kind == 1:                       # two-launch CSR
        C = int(r.integers(17, 513))
        L = n_sink + int(r.integers(max(C, 1100), 4000))
    else:                                 # three-launch CSR
        C = int(r.integers(513, 800))
        L = n_sink + int(r.integers(C, 3500))
    iters = int(r.integers(1, 4))
    return H, n_sink, C, L, iters, dtype


@pytest.mark.parametrize("seed", range(160))
def test_random_decode_shapes(seed):
    cfg = _decode_cfg(seed)
    say(f"random decode shape seed {seed}: H,G,C,Lp,B,sink,pend,dtype = {cfg}")
    fused_case(*cfg)


@pytest.mark.parametrize("seed", range(96))
def test_random_cluster_shapes(seed):
    H, n_sink, C, L, iters, dtype = _cluster_cfg(seed)
    say(f"random cluster shape seed {seed}: H={H} sink={n_sink} C={C} L={L} iters={iters} {dtype}")
    wl = synth.workload(0 if dtype == "f32" else 1)
    K, _, hs = synth.make_kv(wl, L=L, heads=range(H))
    Kf = np.stack([h.Kf for h in hs]).astype(np.float64)
    lloyd_parity(to_dev(K, wl.dtype), Kf, n_sink, C, iters,
                 oracle.EXACT if dtype == "f32" else oracle.MIRROR)
