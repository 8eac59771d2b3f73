"""Whole-layer composition of the oracle steps.  TEST INFRASTRUCTURE ONLY.

A plan row is one (batch b, head h, query block r); rows are numbered
(b*H + h)*QB + r with QB = ceil(N / 128). The plan is kept in CSR form:
rowptr [rows+1] (int64), idx (int32, ascending within each row, original
token order), logw (fp32 log-weights), p (fp64 inclusion probabilities).
[hamidun, "three techniques in AB-Attention", kernel paragraph]: the plan is
rebuilt once every 4 denoising steps and reused by the attention of the
steps in between, so it is a value of its own.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .ibcs import mean_keys, kmeans_block, ibcs_scores_row, query_rows
from .sip import sip_probabilities, draw_row


@dataclass
class OraclePlan:
    B: int
    H: int
    N: int
    d: int
    M: int
    QB: int
    rowptr: np.ndarray
    idx: np.ndarray
    logw: np.ndarray
    p: np.ndarray
    scores: np.ndarray | None = None          # [B, H, QB, M] float64
    centroids: np.ndarray | None = None       # [B, H, QB, C, d] float64
    weights: np.ndarray | None = None         # [B, H, QB, C] float64
    extra: dict = field(default_factory=dict)

    def row(self, b: int, h: int, r: int):
        i = (b * self.H + h) * self.QB + r
        lo, hi = int(self.rowptr[i]), int(self.rowptr[i + 1])
        return self.idx[lo:hi], self.logw[lo:hi], self.p[lo:hi]


def ibcs_scores(Q, K, n_clusters: int = 8, iters: int = 4, query_block: int = 128):
    """IBCS scores for every row of fp64 Q, K [B, H, N, d]."""
    B, H, N, d = Q.shape
    rows = query_rows(N, query_block)
    kbar = mean_keys(K)
    M = kbar.shape[2]
    scores = np.empty((B, H, len(rows), M))
    cents = np.zeros((B, H, len(rows), n_clusters, d))
    wts = np.zeros((B, H, len(rows), n_clusters))
    for b in range(B):
        for h in range(H):
            for r, (lo, hi) in enumerate(rows):
                c, w, _ = kmeans_block(Q[b, h, lo:hi], n_clusters, iters)
                scores[b, h, r] = ibcs_scores_row(c, w, kbar[b, h], d)
                cents[b, h, r] = c
                wts[b, h, r] = w
    return scores, cents, wts


def plan_from_scores(scores32, B: int, H: int, N: int, d: int, budget: int, seed: int,
                     sampling: str = "poisson"):
    """SIP plan from fp32 scores [B, H, QB, M] (sampling: "poisson" or "systematic")."""
    scores32 = np.asarray(scores32, dtype=np.float32)
    QB, M = scores32.shape[2], scores32.shape[3]
    counts = np.zeros(B * H * QB, dtype=np.int64)
    parts = []
    for b in range(B):
        for h in range(H):
            for r in range(QB):
                p = sip_probabilities(scores32[b, h, r], budget)
                parts.append(draw_row(p, seed, b, h, r, sampling))
                counts[(b * H + h) * QB + r] = parts[-1][0].size
    rowptr = np.zeros(B * H * QB + 1, dtype=np.int64)
    rowptr[1:] = np.cumsum(counts)
    idx = np.concatenate([x[0] for x in parts]) if parts else np.zeros(0, np.int32)
    logw = np.concatenate([x[1] for x in parts]) if parts else np.zeros(0, np.float32)
    p = np.concatenate([x[2] for x in parts]) if parts else np.zeros(0)
    return OraclePlan(B, H, N, d, M, QB, rowptr, idx.astype(np.int32),
                      logw.astype(np.float32), p.astype(np.float64))


def build_plan(Q, K, budget: int, seed: int, n_clusters: int = 8, iters: int = 4,
               sampling: str = "poisson"):
    """Full plan: mean keys, IBCS scores, then SIP on the fp32-rounded scores."""
    B, H, N, d = Q.shape
    scores, cents, wts = ibcs_scores(Q, K, n_clusters, iters)
    plan = plan_from_scores(scores.astype(np.float32), B, H, N, d, budget, seed, sampling)
    plan.scores, plan.centroids, plan.weights = scores, cents, wts
    return plan


def plan_attention(Q, K, V, plan: OraclePlan, query_block: int = 128):
    """Horvitz-Thompson attention of every row of fp64 Q, K, V under a plan."""
    from .attention import ht_attention_row
    B, H, N, d = Q.shape
    out = np.zeros(Q.shape[:-1] + (V.shape[-1],))
    for b in range(B):
        for h in range(H):
            for r, (lo, hi) in enumerate(query_rows(N, query_block)):
                idx, logw, _ = plan.row(b, h, r)
                out[b, h, lo:hi] = ht_attention_row(Q[b, h, lo:hi], K[b, h], V[b, h], idx, logw)
    return out
