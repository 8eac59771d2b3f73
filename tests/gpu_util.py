"""Helpers shared by the GPU parity tests: conversions and the acceptance
checks (tolerances as the method's targets state them)."""
from __future__ import annotations

import numpy as np
import torch

import oracle

OUT_REL_L2 = 1e-2      # attention output, given an identical plan
OUT_MAX_ABS = 2e-2
SCORE_REL = 1e-4       # IBCS scores vs the fp64 oracle


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_output(out: np.ndarray, ref: np.ndarray, what: str = ""):
    diff = out - ref
    rel = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)
    mx = float(np.abs(diff).max()) if diff.size else 0.0
    assert rel <= OUT_REL_L2 and mx <= OUT_MAX_ABS, f"{what}: rel L2 {rel:.3e}, max abs {mx:.3e}"
    return rel, mx


def score_error(s_gpu: np.ndarray, s_ref: np.ndarray) -> np.ndarray:
    """Per-row max_j |s_gpu - s_ref| / max(s_ref_j, 1e-6 * max_j s_ref)."""
    s_gpu = s_gpu.reshape(-1, s_gpu.shape[-1]).astype(np.float64)
    s_ref = s_ref.reshape(-1, s_ref.shape[-1])
    floor = 1e-6 * s_ref.max(axis=1, keepdims=True)
    return (np.abs(s_gpu - s_ref) / np.maximum(s_ref, floor)).max(axis=1)


def ulp_diff_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ai = a.astype(np.float32).view(np.int32).astype(np.int64)
    bi = b.astype(np.float32).view(np.int32).astype(np.int64)
    return np.abs(ai - bi)


def check_plan_exact(gp: dict, op: oracle.OraclePlan, what: str = ""):
    """Row pointers, indices and p bit-exact; log-weights within 1 fp32 ulp."""
    np.testing.assert_array_equal(gp["rowptr"], op.rowptr, err_msg=f"{what}: rowptr")
    np.testing.assert_array_equal(gp["idx"], op.idx, err_msg=f"{what}: idx")
    assert np.array_equal(gp["p"].view(np.uint64), op.p.view(np.uint64)), f"{what}: p not bit-exact"
    u = ulp_diff_f32(gp["logw"], op.logw)
    assert (u <= 1).all(), f"{what}: logw off by {u.max()} ulp"
    return int((u == 1).sum())


def oracle_plan_of(gp: dict, B, H, N, d) -> oracle.OraclePlan:
    M, QB = N // 4, (N + 127) // 128
    return oracle.OraclePlan(B, H, N, d, M, QB, gp["rowptr"], gp["idx"], gp["logw"], gp["p"])


# Relative margin (second-nearest minus nearest squared distance, over the
# nearest) below which an assignment may go either way: the oracle sums
# (q - c)^2 and the kernel |c|^2 - 2 q.c, both in fp64, and their rounding
# differs by a few units of 2^-52 of |q|^2 + |c|^2, far below this.
KMEANS_TIE_REL = 1e-12
CENT_TOL = 1e-6        # centroids: fp32 rounding of the fp64 member means


def _cluster_match(w_gpu, c_gpu, w_ref, c_ref):
    return (np.array_equal(w_gpu, w_ref.astype(np.float32)) and
            np.abs(c_gpu - c_ref).max() <= CENT_TOL * max(1.0, float(np.abs(c_ref).max())))


def clustering_references(Q64, w_gpu, c_gpu, ref_w, ref_c, N, C, T, what=""):
    """The oracle clustering each row of the GPU's result equals.

    A row matches the plain oracle run when its weights are the same fp32
    values (counts over n) and its centroids lie within fp32 rounding of the
    oracle's member means. A row that does not is accepted only if the
    oracle saw a near-tie (relative margin below KMEANS_TIE_REL) and the GPU's
    weights and centroids equal the oracle run with that decision taken the
    other way (oracle.kmeans_tie_variants): then they are the counts and
    member means of an assignment the rule admits. Asserts that every row
    matches; returns (weights [rows, C], centroids [rows, C, d]) of the
    matching runs and the list of flipped rows. Prints the number of flips.
    """
    B, H = Q64.shape[0], Q64.shape[1]
    QB = (N + 127) // 128
    rows = B * H * QB
    w_gpu = w_gpu.reshape(rows, C)
    c_gpu = c_gpu.reshape(rows, C, -1)
    out_w = ref_w.reshape(rows, C).copy()
    out_c = ref_c.reshape(rows, C, -1).copy()
    flipped = []
    for row in range(rows):
        if _cluster_match(w_gpu[row], c_gpu[row], out_w[row], out_c[row]):
            continue
        bh, r = divmod(row, QB)
        b, h = divmod(bh, H)
        lo, hi = r * 128, min(r * 128 + 128, N)
        variants = oracle.kmeans_tie_variants(Q64[b, h, lo:hi], C, T, KMEANS_TIE_REL)
        hit = [v for v in variants[1:] if _cluster_match(w_gpu[row], c_gpu[row], v[1], v[0])]
        assert hit, (f"{what}: row {row} clusters differ from the oracle's and from every "
                     f"near-tie variant ({len(variants) - 1} variants)")
        out_c[row], out_w[row] = hit[0][0], hit[0][1]
        flipped.append(row)
    print(f"{what}: rows whose k-means took the other side of a near-tie: {len(flipped)} "
          f"of {rows}")
    return out_w, out_c, flipped


def row_clustering_reference(Qr, w_gpu, c_gpu, C, T, what=""):
    """clustering_references for one row given its queries Qr [n, d]:
    returns (centroids, weights, flipped)."""
    variants = oracle.kmeans_tie_variants(Qr, C, T, KMEANS_TIE_REL)
    for i, (c, w, _) in enumerate(variants):
        if _cluster_match(w_gpu.reshape(C), c_gpu.reshape(C, -1), w, c):
            return c, w, i > 0
    raise AssertionError(f"{what}: clusters differ from the oracle's and from every near-tie "
                         f"variant ({len(variants) - 1} variants)")


def reference_scores(K64, ref_w, ref_c, rows_idx, N, H):
    """Oracle scores of the given rows from the given clusterings."""
    QB = (N + 127) // 128
    d = K64.shape[-1]
    out = {}
    kb = {}
    for row in rows_idx:
        bh, r = divmod(int(row), QB)
        b, h = divmod(bh, H)
        if (b, h) not in kb:
            kb[(b, h)] = oracle.mean_keys(K64[b, h])
        out[int(row)] = oracle.ibcs_scores_row(ref_c[row], ref_w[row], kb[(b, h)], d)
    return out
