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
