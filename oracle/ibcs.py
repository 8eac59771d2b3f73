"""IBCS (intra-block clustering selector) in fp64.  TEST INFRASTRUCTURE ONLY.

[hamidun, "three techniques in AB-Attention", IBCS paragraph]: queries are cut
into blocks of 128 tokens; inside each block they are grouped into 8 clusters,
each carrying a centroid and a weight equal to its share of the block's
queries; a KV block is scored by the weighted attention of the centroids
toward the block's averaged keys. The clusters serve only the estimate: the
tokens are never reordered ([edumints, "three innovations", IBCS item]).

Readings where the pages are silent:
  * clustering = Lloyd (batch) k-means run for a fixed number of iterations T;
  * initial centroids = evenly strided queries of the block, q[floor(m*n/C)];
  * distance = squared Euclidean on the raw query vectors; ties go to the
    smallest cluster index; an empty cluster keeps its centroid and gets
    weight 0;
  * a partial last block clusters only its n < 128 real queries, with
    C_eff = min(C, n) clusters;
  * "averaged keys" = arithmetic mean of the 4 keys of a KV block;
  * score of KV block j: s_j = sum_m w_m softmax_j(c_m . kbar_j / sqrt(d)),
    the softmax running over all M KV blocks of the same (batch, head).
"""
from __future__ import annotations

import math

import numpy as np


def query_rows(N: int, query_block: int = 128):
    """Row r covers queries [r*Bq, min((r+1)*Bq, N)); returns a list of (lo, hi)."""
    return [(lo, min(lo + query_block, N)) for lo in range(0, N, query_block)]


def mean_keys(K: np.ndarray, kv_block: int = 4) -> np.ndarray:
    """Averaged key of every KV block: kbar_j = (1/4) * sum_{t<4} k_{4j+t}.

    K: [..., N, d] float64 with N a multiple of kv_block. Returns [..., N/4, d].
    """
    N, d = K.shape[-2], K.shape[-1]
    if N % kv_block:
        raise ValueError("N must be a multiple of the KV block size")
    grouped = K.reshape(*K.shape[:-2], N // kv_block, kv_block, d)
    total = grouped.sum(axis=-2)
    return total / kv_block


def kmeans_block(Qr: np.ndarray, n_clusters: int = 8, iters: int = 4,
                 return_margin: bool = False, override: dict | None = None,
                 trace: list | None = None):
    """Lloyd k-means on the queries of one query block, in their original order.

    Qr: [n, d] float64 (n >= 1). Returns (centroids [C, d], weights [C],
    assignment [n]) where C = n_clusters; clusters beyond C_eff = min(C, n)
    are zero with weight 0. Weights are the clusters' shares of the block's
    queries under the last assignment, and the centroids are the means of
    that same assignment. With return_margin, a fourth value gives the
    smallest relative gap (second-nearest minus nearest, over nearest) seen
    in any assignment step: a gap near rounding level marks a decision that
    another summation order may take the other way.

    override maps (iteration, query) to a cluster that the assignment of
    that query in that iteration takes instead of its nearest one; trace, a
    list, receives the [n, C_eff] squared distances of every iteration.
    Both only serve kmeans_tie_variants; the default result ignores them.
    """
    n, d = Qr.shape
    if n < 1 or iters < 1 or n_clusters < 1:
        raise ValueError("need n >= 1, iters >= 1, n_clusters >= 1")
    c_eff = min(n_clusters, n)
    start = [(m * n) // c_eff for m in range(c_eff)]
    cent = Qr[start].copy()
    assign = np.zeros(n, dtype=np.int64)
    margin = np.inf
    for it in range(iters):
        diff = Qr[:, None, :] - cent[None, :, :]           # [n, C_eff, d]
        dist2 = np.einsum("ncd,ncd->nc", diff, diff)
        assign = np.argmin(dist2, axis=1)                  # first minimum wins
        if trace is not None:
            trace.append(dist2)
        if override:
            for (oit, i), m in override.items():
                if oit == it:
                    assign[i] = m
        if return_margin and c_eff > 1:
            srt = np.sort(dist2, axis=1)
            gap = (srt[:, 1] - srt[:, 0]) / np.maximum(srt[:, 0], 1e-300)
            margin = min(margin, float(gap.min()))
        for m in range(c_eff):
            members = assign == m
            cnt = int(members.sum())
            if cnt:
                cent[m] = Qr[members].sum(axis=0) / cnt
    counts = np.bincount(assign, minlength=c_eff).astype(np.float64)
    centroids = np.zeros((n_clusters, d))
    centroids[:c_eff] = cent
    weights = np.zeros(n_clusters)
    weights[:c_eff] = counts / n
    if return_margin:
        return centroids, weights, assign, margin
    return centroids, weights, assign


def ibcs_scores_row(centroids: np.ndarray, weights: np.ndarray, kbar: np.ndarray,
                    d: int | None = None) -> np.ndarray:
    """Score every KV block for one query block.

    s_j = sum_m w_m * exp(x_mj - max_j x_mj) / sum_j exp(x_mj - max_j x_mj),
    x_mj = c_m . kbar_j / sqrt(d). Clusters with weight 0 add nothing.
    Returns [M] float64; the entries are >= 0 and sum to 1.
    """
    if d is None:
        d = kbar.shape[-1]
    x = centroids @ kbar.T / math.sqrt(d)                 # [C, M]
    x = x - x.max(axis=1, keepdims=True)
    e = np.exp(x)
    pi = e / e.sum(axis=1, keepdims=True)
    return weights @ pi


def ibcs_row(Qr: np.ndarray, kbar: np.ndarray, n_clusters: int = 8, iters: int = 4):
    """k-means then scores for one query block; returns (scores, centroids, weights)."""
    cent, w, _ = kmeans_block(Qr, n_clusters, iters)
    return ibcs_scores_row(cent, w, kbar, Qr.shape[1]), cent, w


def kmeans_tie_variants(Qr: np.ndarray, n_clusters: int = 8, iters: int = 4,
                        rel_tol: float = 1e-12, limit: int = 64):
    """Every result the Lloyd iteration of kmeans_block reaches when each
    assignment decided by a near-tie may go either way.

    A query whose two nearest centroids lie within a relative gap rel_tol of
    each other ((second - nearest) / nearest) has a decision that another
    summation order can take the other way, with either outcome a correct
    reading of the rule. Starting from the plain run, each such decision
    (taken in order of iteration, then query) is branched to the
    second-nearest cluster and the iteration re-run from it. Returns a list
    of (centroids, weights, override) with the plain result first, at most
    `limit` entries.
    """
    out = []
    stack = [{}]
    while stack and len(out) < limit:
        ov = stack.pop()
        trace = []
        cent, w, _ = kmeans_block(Qr, n_clusters, iters, override=ov, trace=trace)
        out.append((cent, w, dict(ov)))
        last = max(ov) if ov else (-1, -1)
        for it, dist2 in enumerate(trace):
            if dist2.shape[1] < 2 or it < last[0]:
                continue
            order = np.argsort(dist2, axis=1, kind="stable")
            near = dist2[np.arange(dist2.shape[0]), order[:, 0]]
            second = dist2[np.arange(dist2.shape[0]), order[:, 1]]
            gap = (second - near) / np.maximum(near, 1e-300)
            for i in np.nonzero(gap < rel_tol)[0]:
                key = (it, int(i))
                if key <= last:
                    continue
                branch = dict(ov)
                branch[key] = int(order[i, 1])
                stack.append(branch)
    return out
