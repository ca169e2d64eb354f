"""Helpers shared by the GPU parity tests (no test functions here)."""
import sys

import numpy as np
import torch

import oracle
import sparse_decode_attention_ckv_amd as ck
import synth

DEV = "cuda:0"


def say(msg: str):
    """Name the case before each GPU step, flushed, so a failing run's last
    line identifies it."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(storage: np.ndarray, dtype: str) -> torch.Tensor:
    """synth storage array (float32 or uint16 bf16 bits) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(storage).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(storage, dtype=np.float32))
    return t.to(DEV)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(o: np.ndarray, ref: np.ndarray) -> float:
    """max over query heads of max|o - ref| / max|ref| (per head)."""
    worst = 0.0
    for h in range(ref.shape[0]):
        den = np.abs(ref[h]).max()
        num = np.abs(o[h] - ref[h]).max()
        worst = max(worst, num / den if den > 0 else num)
    return worst


def gpu_cluster(K, n_sink, C, iters, **kw):
    out = ck.ckv_cluster(K, n_sink, C, iters, **kw)
    torch.cuda.synchronize()
    return out


# Label parity margin of the cosine assignment, in cosine units (the
# oracle's cosine margins are): the tolerance the assignment is held to.
# The bf16 kernel's own error is far below it: fp32 accumulation of exact
# bf16 products, and an argmax that compares 2|k| + <k, mu~> truncated to
# 2^-18 of its magnitude (1.2e-5 |k| at most, 1.2e-5 in cosine units).
ASSIGN_MARGIN = 1e-4

# the library's metric codes for the oracle's
CK_METRIC = {oracle.COSINE: ck.CKV_COSINE, oracle.INNER_PRODUCT: ck.CKV_INNER_PRODUCT,
             oracle.L2: ck.CKV_L2}


def margin_threshold(metric, Kw, mu, labels, margin, mode):
    """Per-token margin below which a label is not compared. Cosine margins
    are in cosine units: the absolute `margin`. Inner-product and L2 scores are
    unbounded and compared exactly by the kernel, so the threshold is the
    worst-case fp32 accumulation error of two scores (the operands as the
    kernel reads them: mu rounded to bf16 under MIRROR): 128 products, each
    sum rounded, 128 * 2^-24 |k| max|mu| per score; twice the score gap
    plus the bias rounding for the L2 squared-distance gap; a safety factor
    of 2 over all."""
    if metric == oracle.COSINE:
        return margin
    mu_r = mu if mode == oracle.EXACT else synth.bf16_to_f32(synth.bf16_bits(mu)).astype(
        np.float64)
    kn = np.linalg.norm(Kw, axis=1)
    M = np.linalg.norm(mu_r, axis=1).max()
    gap = 2 * 128 * 2.0 ** -24 * kn * M
    if metric == oracle.L2:
        gap = 2 * gap + 2.0 ** -22 * M * M
    return 2 * gap


def lloyd_parity(Kdev, Kf64, n_sink, C, iters, mode, tol_mu=1e-4, margin=ASSIGN_MARGIN,
                 token_base=0, sample=None, metric=oracle.COSINE):
    """Per-iteration parity of the GPU K-means against the oracle.

    For t = 1..iters the GPU runs t iterations from scratch (a prefix of the
    same deterministic sequence). The oracle starts iteration t from the
    GPU's centroids of iteration t-1 and must reproduce:
      * labels, bit-exact, for tokens whose top-2 margin is >= `margin`
        (ASSIGN_MARGIN; scaled per token for inner product and L2);
      * the CSR of the GPU's labels, bit-exact;
      * the centroids of the GPU's labels, max abs error <= tol_mu.
    Kf64: [H][L][d] exact values. `sample`: optional token subset (window
    rows >= n_sink) for the label check at large sizes. `metric` is the
    oracle's assignment distance (the GPU runs the same one).
    Returns per-iteration (excluded fraction) list."""
    H, L, d = Kf64.shape
    Lp = L - n_sink
    mu_prev = np.stack([oracle.init_centroids(Kf64[h], n_sink, C) for h in range(H)])
    excluded = []
    for t in range(1, iters + 1):
        say(f"  lloyd iteration {t}/{iters} (H={H}, L={L}, C={C})")
        cent, asg, off, tok = gpu_cluster(Kdev, n_sink, C, t, token_base=token_base,
                                          metric=CK_METRIC[metric])
        mu_g = host_f64(cent)
        a_g = asg.cpu().numpy()
        off_g = off.cpu().numpy()
        tok_g = tok.cpu().numpy()
        assert np.all(a_g[:, :n_sink] == -1)
        ex = 0
        for h in range(H):
            if sample is None:
                a_o, m_o = oracle.assign(Kf64[h], n_sink, mu_prev[h], mode=mode, metric=metric)
                keep = m_o[n_sink:] >= margin_threshold(metric, Kf64[h][n_sink:], mu_prev[h],
                                                        a_o[n_sink:], margin, mode)
                got = a_g[h, n_sink:]
                want = a_o[n_sink:]
            else:
                a_o, m_o = oracle.assign(Kf64[h][sample], 0, mu_prev[h], mode=mode,
                                         metric=metric)
                keep = m_o >= margin_threshold(metric, Kf64[h][sample], mu_prev[h], a_o, margin,
                                               mode)
                got = a_g[h, sample]
                want = a_o
            bad = np.nonzero(keep & (got != want))[0]
            assert bad.size == 0, (t, h, bad[:10], got[bad[:10]], want[bad[:10]])
            ex += int((~keep).sum())
            o_off, o_tok = oracle.csr(a_g[h], n_sink, C, token_base=token_base)
            assert np.array_equal(off_g[h], o_off), (t, h)
            assert np.array_equal(tok_g[h], o_tok), (t, h)
            mu_o = oracle.update(Kf64[h], n_sink, a_g[h], mu_prev[h], mode=mode)
            err = np.abs(mu_g[h] - mu_o).max()
            assert err <= tol_mu, (t, h, err)
        excluded.append(ex / (H * (Lp if sample is None else len(sample))))
        mu_prev = mu_g
    return excluded
