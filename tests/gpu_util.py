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


def flips_explained(Q64, rows_bad, N, C, T, margin_tol=1e-9):
    """True if every row whose cluster weights differ had a near-tie in the
    oracle's assignment (so either side's decision is a correct reading)."""
    B, H = Q64.shape[0], Q64.shape[1]
    QB = (N + 127) // 128
    for row in rows_bad:
        bh, r = divmod(int(row), QB)
        b, h = divmod(bh, H)
        lo, hi = r * 128, min(r * 128 + 128, N)
        *_, margin = oracle.kmeans_block(Q64[b, h, lo:hi], C, T, return_margin=True)
        if margin > margin_tol:
            return False
    return True
