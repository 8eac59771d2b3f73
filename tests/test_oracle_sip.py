"""Pins of the oracle's SIP probabilities, Philox generator and draws (CPU only)."""
import numpy as np
import pytest

import oracle
from tests.conftest import load_golden


def test_philox_known_answers():
    for v in load_golden("philox_kat.yaml")["vectors"]:
        out = oracle.philox4x32_10(*v["counter"], *v["key"])
        assert [int(x) for x in out] == v["out"]


def test_philox_vectorised_matches_scalar_calls():
    j = np.arange(37, dtype=np.uint64)
    vec = oracle.philox4x32_10(j, 3, 5, 7, 11, 13)
    for i in (0, 17, 36):
        one = oracle.philox4x32_10(i, 3, 5, 7, 11, 13)
        assert [int(x[i]) for x in vec] == [int(x) for x in one]


def test_uniforms_are_uniform():
    u = oracle.sip_uniforms(seed=0x5EED0000, b=0, h=3, r=7, M=200000)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / u.size)
    hist = np.histogram(u, bins=20, range=(0, 1))[0]
    exp = u.size / 20
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert chi2 < 60          # 19 dof; p < 1e-5 beyond this
    # distinct counters give distinct streams
    u2 = oracle.sip_uniforms(seed=0x5EED0000, b=0, h=3, r=8, M=1000)
    assert not np.array_equal(u[:1000], u2)


@pytest.mark.parametrize("i", range(9))
def test_probabilities_hand_examples(i):
    g = load_golden("sip_examples.yaml")["examples"][i]
    p = oracle.sip_probabilities(np.array(g["scores"], dtype=np.float32), g["budget"])
    if g["exact"]:
        np.testing.assert_array_equal(p, np.array(g["p"]))
    else:
        np.testing.assert_allclose(p, np.array(g["p"]), rtol=0, atol=1e-7)


def _random_scores(rng, M, kind):
    if kind == "dirichlet":
        s = rng.dirichlet(np.full(M, 0.3))
    elif kind == "peaked":
        s = np.exp(rng.standard_normal(M) * 3)
        s /= s.sum()
    else:
        s = np.full(M, 1.0 / M)
    return s.astype(np.float32)


@pytest.mark.parametrize("kind", ["dirichlet", "peaked", "flat"])
@pytest.mark.parametrize("M,K", [(256, 64), (256, 1), (2048, 205), (512, 511), (300, 300)])
def test_probability_invariants(kind, M, K):
    rng = np.random.default_rng(M + K)
    s = _random_scores(rng, M, kind)
    p = oracle.sip_probabilities(s, K)
    assert (p >= 0).all() and (p <= 1).all()
    assert abs(p.sum() - K) <= 1e-12 * K
    # p is non-decreasing in s
    order = np.argsort(s, kind="stable")
    assert (np.diff(p[order]) >= 0).all()
    # below the cap, p is proportional to s
    # (scores enter as floor(s * 2^52), so proportionality is exact up to an
    # absolute c * 2^-52 per block)
    free = (p < 1) & (s > 0)
    if free.sum() > 1:
        top = np.argmax(np.where(free, s, -1.0))
        c = p[top] / float(s[top])
        err = np.abs(p[free] - c * s[free].astype(np.float64))
        assert err.max() <= c * 2.0 ** -51 + 4e-16
    # capped blocks are the highest-scoring ones
    if (p == 1).any() and (p < 1).any():
        assert s[p == 1].min() >= s[p < 1].max()
    if K == M:
        assert (p == 1).all()


def test_probabilities_reject_bad_input():
    with pytest.raises(ValueError):
        oracle.sip_probabilities(np.array([0.5, 0.5], np.float32), 0)
    with pytest.raises(ValueError):
        oracle.sip_probabilities(np.array([0.5, 0.5], np.float32), 3)
    with pytest.raises(ValueError):
        oracle.sip_probabilities(np.array([1.0, 1.0, 0.5], np.float32), 1)
    with pytest.raises(ValueError):
        oracle.sip_probabilities(np.array([-0.1, 0.5], np.float32), 1)


def test_quarter_probability_gives_ln4_offset():
    g = load_golden("sip_examples.yaml")
    # find a seed whose draw keeps the single block at p = 1/4
    for seed in range(100):
        idx, logw, p = oracle.sip_draw_row(np.array([0.25]), seed, 0, 0, 0)
        if idx.size:
            break
    assert idx.size == 1 and p[0] == 0.25
    assert float(logw[0]) == g["quarter_logw_fp32"]
    idx, logw, p = oracle.sip_draw_row(np.array([1.0, 0.0]), 1, 0, 0, 0)
    assert list(idx) == [0] and logw[0] == 0.0 and not np.signbit(logw[0])


def test_draw_frequencies_match_probabilities():
    rng = np.random.default_rng(12)
    M, K, S = 64, 12, 4000
    s = _random_scores(rng, M, "peaked")
    p = oracle.sip_probabilities(s, K)
    hits = np.zeros(M)
    counts = np.zeros(S)
    for seed in range(S):
        idx, logw, pk = oracle.sip_draw_row(p, seed, 0, 1, 2)
        assert (np.diff(idx) > 0).all()                 # ascending, no repeats
        np.testing.assert_array_equal(pk, p[idx])
        hits[idx] += 1
        counts[seed] = idx.size
    assert (hits[p == 1] == S).all()
    z = (hits - S * p) / np.sqrt(np.maximum(S * p * (1 - p), 1e-300))
    assert np.abs(z[(p > 0) & (p < 1)]).max() < 5
    var = (p * (1 - p)).sum()
    assert abs(counts.mean() - K) < 5 * np.sqrt(var / S)
    assert abs(counts.var() / var - 1) < 0.15


# ---- fixed-size (systematic) design --------------------------------------

def _u_grid(n=4096):
    """n evenly spaced values of U covering [0, 2^40)."""
    return [t * (oracle.sip.SYS_UNIT // n) for t in range(n)]


def test_systematic_inclusion_counts_over_u_grid():
    """Over U on an even grid of 4096 points, block j must be taken for
    P_j / 2^28 of them, give or take one: its inclusion probability is
    exactly P_j 2^-40. A wrong cumulative sum (inclusive for exclusive), an
    off-by-one in the point count or a lost carry shows up here."""
    p = np.array([0.3, 1.0, 0.05, 0.65, 2.0 ** -30, 0.0, 0.999999, 1.0, 0.25, 0.7500001])
    P = oracle.systematic_sizes(p)
    grid = _u_grid()
    hits = np.zeros(p.size, dtype=np.int64)
    for U in grid:
        hits += oracle.systematic_select(P, U)
    expect = P.astype(np.float64) / float(oracle.sip.SYS_UNIT // len(grid))
    assert np.all(np.abs(hits - expect) <= 1.0), (hits, expect)
    assert hits[1] == hits[7] == len(grid)            # p = 1: always taken
    assert hits[5] == 0                                # p = 0: never


def test_systematic_equal_sizes_closed_form():
    """p = 1/4 on 64 blocks (sum 16 exactly): the sample is every fourth
    block starting at floor(U / 2^38), for any U."""
    p = np.full(64, 0.25)
    P = oracle.systematic_sizes(p)
    rng = np.random.default_rng(3)
    for U in list(rng.integers(0, oracle.sip.SYS_UNIT, size=50)) + [0, oracle.sip.SYS_UNIT - 1]:
        U = int(U)
        sel = np.nonzero(oracle.systematic_select(P, U))[0]
        j0 = U >> 38
        np.testing.assert_array_equal(sel, np.arange(j0, 64, 4))


def test_systematic_sample_size_is_the_budget():
    """Rows from the capped water-filling (sum of p = K up to rounding):
    every draw takes K blocks, or K - 1 / K + 1 when rounding moved the
    fixed-point total off K 2^40, and then only if U falls in that gap."""
    rng = np.random.default_rng(11)
    for t in range(40):
        M = int(rng.integers(50, 400))
        K = int(rng.integers(1, M + 1))
        s = rng.random(M) ** rng.uniform(1, 8)
        s32 = (s / s.sum() * 0.999).astype(np.float32)
        p = oracle.sip_probabilities(s32, K)
        P = oracle.systematic_sizes(p)
        total = int(P.sum(dtype=np.uint64))
        idx, logw, pk = oracle.systematic_draw_row(p, 1234 + t, 0, t % 3, t)
        lo, hi = total >> 40, -(-total >> 40)
        assert lo <= idx.size <= hi, (idx.size, lo, hi)
        assert K - 1 <= idx.size <= K + 1
        assert np.all(np.diff(idx) > 0)
        assert np.array_equal(pk, P[idx].astype(np.float64) * 2.0 ** -40)
        assert np.all((p[idx] == 1.0) == (pk == 1.0))


def test_systematic_capped_blocks_always_taken_and_unbiased_total():
    """Every p = 1 block is in every sample; the Horvitz-Thompson total of a
    fixed vector, averaged over the U grid, equals its true total (each
    block is counted P_j/2^28 times out of 4096, weighted by 2^40/P_j)."""
    rng = np.random.default_rng(5)
    s = rng.random(300) ** 6
    s[[7, 100, 250]] = 40.0                          # three blocks certain to be capped
    p = oracle.sip_probabilities((s / s.sum() * 0.999).astype(np.float32), 40)
    assert (p == 1.0).sum() > 0
    P = oracle.systematic_sizes(p)
    x = rng.standard_normal(300)
    grid = _u_grid()
    est = 0.0
    for U in grid:
        sel = oracle.systematic_select(P, U)
        assert sel[p == 1.0].all()
        est += (x[sel] * (float(oracle.sip.SYS_UNIT) / P[sel].astype(np.float64))).sum()
    est /= len(grid)
    # each block's count is within one of its expectation: error <= sum |x_j| 2^40/(P_j 4096)
    bound = (np.abs(x[P > 0]) * float(oracle.sip.SYS_UNIT) / (P[P > 0].astype(np.float64) * len(grid))).sum()
    assert abs(est - x[P > 0].sum()) <= bound + 1e-9


def test_systematic_uniform_range_and_row_dependence():
    us = {oracle.systematic_uniform(99, b, h, r) for b in range(2) for h in range(3) for r in range(5)}
    assert len(us) == 30 and all(0 <= u < oracle.sip.SYS_UNIT for u in us)
