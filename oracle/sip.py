"""SIP (sampling with inclusion-probability weighting) in fp64.  TEST INFRASTRUCTURE ONLY.

[hamidun, "three techniques in AB-Attention", SIP paragraph]: a KV block joins
the sample with probability proportional to its score; the most important
blocks are always taken and every other block keeps a non-zero chance; each
chosen block is weighted by the inverse of its inclusion probability (a block
taken with p = 25% counts four times), which is the Horvitz-Thompson
estimator and leaves both the softmax numerator and its normaliser unbiased;
the result is ordinary softmax attention on shifted logits, so no correction
pass is needed. [edumints, "three innovations", SIP item] says the same.

Readings where the pages are silent:
  * probabilities p_j = min(1, c * s_j) with c chosen so that sum_j p_j equals
    the budget K (KV blocks per query block); blocks whose p reaches 1 are the
    "always taken" ones. c is found by capped water-filling, in fixed point so
    that every sum is exact and independent of summation order:
      q_j = floor(s_j * 2^52) as an integer (s_j is the fp32 score in [0, 1],
      and the row of scores sums to at most 2, so sum q_j < 2^53);
      U = all blocks, t = 0; repeat:
        if K - t >= |U|: p = 1 on U, stop;
        S = sum_{U} q_j; if S == 0: p = (K - t)/|U| on U, stop;
        c = (K - t) / S  (IEEE double division);
        Z = {j in U : c * q_j >= 1} (IEEE double product);
        if Z is empty: p_j = c * q_j on U, stop;
        p = 1 on Z, t += |Z|, U -= Z.
  * sampling design = Poisson: one independent Bernoulli(p_j) per block, so
    the count per row varies around K; the draw uses one uniform per block
    from Philox4x32-10(key = (seed_lo, seed_hi), counter = (j >> 1, r, h, b)):
    one call yields four 32-bit words (x0, x1, x2, x3), block 2i takes
    (hi, lo) = (x0, x1) and block 2i+1 takes (x2, x3), u = ((hi << 32 | lo)
    >> 11) * 2^-53, and block j is kept iff u < p_j;
  * the Horvitz-Thompson weight 1/p enters as the logit offset
    logw = -ln(p) (natural log, fp64, rounded to fp32; +0 for p = 1).
  * a second, fixed-size design (the pages speak of a fixed budget per query
    block; the Poisson design meets it only in expectation): systematic
    sampling with unequal probabilities. In fixed point with unit 2^-40,
    P_j = floor(p_j * 2^40); C_j = P_0 + ... + P_j (exact integers); one
    uniform U in [0, 2^40) per row, from Philox4x32-10(key = seed, counter =
    (2^32 - 1, r, h, b)), words (x0, x1) as (hi, lo), U = (hi << 32 | lo) >> 24;
    the points U + k 2^40 (k = 0, 1, ...) fall in the intervals [C_{j-1}, C_j),
    and block j is taken iff its interval holds one. Block j is then taken
    with probability exactly P_j 2^-40 (its interval is at most 2^40 long),
    which is the p the plan records and weights by; the row takes
    floor or ceil of sum P / 2^40 blocks, i.e. K, or K - 1 when rounding left
    the sum just below K 2^40 and U fell in the gap.
"""
from __future__ import annotations

import numpy as np

from .philox import philox4x32_10

TWO52 = float(2 ** 52)


def fixed_point_scores(s32: np.ndarray) -> np.ndarray:
    """q_j = floor(s_j * 2^52) for fp32 scores in [0, 1], as uint64."""
    s = np.asarray(s32, dtype=np.float32).astype(np.float64)
    if np.any(~np.isfinite(s)) or np.any(s < 0.0) or np.any(s > 1.0):
        raise ValueError("scores must lie in [0, 1]")
    return np.floor(s * TWO52).astype(np.uint64)


def sip_probabilities(s32: np.ndarray, budget: int) -> np.ndarray:
    """Capped inclusion probabilities of one row; returns float64 [M]."""
    q = fixed_point_scores(s32)
    M = q.shape[0]
    if not 1 <= budget <= M:
        raise ValueError("budget must lie in [1, M]")
    if int(q.sum(dtype=np.uint64)) >= 2 ** 53:
        raise ValueError("a row of scores must sum to less than 2")
    p = np.zeros(M, dtype=np.float64)
    active = np.ones(M, dtype=bool)
    taken = 0
    while True:
        n_active = int(active.sum())
        left = budget - taken
        if left >= n_active:
            p[active] = 1.0
            return p
        S = int(q[active].sum(dtype=np.uint64))
        if S == 0:
            p[active] = float(left) / float(n_active)
            return p
        c = float(left) / float(S)
        act_idx = np.nonzero(active)[0]
        prod = c * q[act_idx].astype(np.float64)
        capped = prod >= 1.0
        if not capped.any():
            p[act_idx] = prod
            return p
        hit = act_idx[capped]
        p[hit] = 1.0
        active[hit] = False
        taken += int(hit.size)


def sip_uniforms(seed: int, b: int, h: int, r: int, M: int) -> np.ndarray:
    """u_j in [0, 1) for j < M: Philox4x32-10 with key = seed and counter
    (j >> 1, r, h, b); even j takes output words 0 and 1, odd j words 2 and 3."""
    j = np.arange(M, dtype=np.uint64)
    x0, x1, x2, x3 = philox4x32_10(j >> np.uint64(1), r, h, b, seed & 0xFFFFFFFF,
                                   (seed >> 32) & 0xFFFFFFFF)
    odd = (j & np.uint64(1)).astype(bool)
    hi = np.where(odd, x2, x0)
    lo = np.where(odd, x3, x1)
    u53 = ((hi << np.uint64(32)) | lo) >> np.uint64(11)
    return u53.astype(np.float64) * (2.0 ** -53)


def sip_draw_row(p: np.ndarray, seed: int, b: int, h: int, r: int):
    """Poisson draw of one row: ascending kept block indices, fp32 log-weights, p."""
    u = sip_uniforms(seed, b, h, r, p.shape[0])
    keep = np.nonzero(u < p)[0]
    pk = p[keep]
    logw = np.where(pk == 1.0, 0.0, -np.log(pk)).astype(np.float32)
    return keep.astype(np.int32), logw, pk


SYS_BITS = 40
SYS_UNIT = 1 << SYS_BITS


def systematic_uniform(seed: int, b: int, h: int, r: int) -> int:
    """The row's U in [0, 2^40) for the fixed-size design."""
    x0, x1, _, _ = philox4x32_10(np.array([0xFFFFFFFF], dtype=np.uint64), r, h, b,
                                 seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    return int(((int(x0[0]) << 32) | int(x1[0])) >> 24)


def systematic_sizes(p: np.ndarray) -> np.ndarray:
    """P_j = floor(p_j * 2^40) as uint64 (p in [0, 1])."""
    return np.floor(np.asarray(p, dtype=np.float64) * float(SYS_UNIT)).astype(np.uint64)


def systematic_select(P: np.ndarray, U: int) -> np.ndarray:
    """Blocks whose interval [C_{j-1}, C_j) holds a point U + k 2^40 (k >= 0)."""
    P = np.asarray(P, dtype=np.uint64)
    C = np.cumsum(P, dtype=np.uint64)
    Cprev = C - P
    U = np.uint64(U)

    def points_below(x):
        # #{k >= 0 : U + k 2^40 < x}
        above = x > U
        safe = np.where(above, x - U - np.uint64(1), np.uint64(0))
        return np.where(above, (safe >> np.uint64(SYS_BITS)) + np.uint64(1), np.uint64(0))

    return points_below(C) > points_below(Cprev)


def systematic_draw_row(p: np.ndarray, seed: int, b: int, h: int, r: int):
    """Fixed-size draw of one row: ascending kept block indices, fp32
    log-weights -ln(P 2^-40), and the inclusion probabilities P 2^-40."""
    P = systematic_sizes(p)
    keep = np.nonzero(systematic_select(P, systematic_uniform(seed, b, h, r)))[0]
    pk = P[keep].astype(np.float64) * (1.0 / SYS_UNIT)
    logw = np.where(pk == 1.0, 0.0, -np.log(pk)).astype(np.float32)
    return keep.astype(np.int32), logw, pk


def draw_row(p: np.ndarray, seed: int, b: int, h: int, r: int, sampling: str = "poisson"):
    """The row's draw under the named design ("poisson" or "systematic")."""
    if sampling == "poisson":
        return sip_draw_row(p, seed, b, h, r)
    if sampling == "systematic":
        return systematic_draw_row(p, seed, b, h, r)
    raise ValueError(f"unknown sampling design {sampling!r}")
