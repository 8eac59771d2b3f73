"""Pins of the oracle's layer-level composition (plan row numbering, the
head and query-block indexing of the scores) and of the Philox word layout
of the draws, against values fixed outside the oracle: the published
Philox4x32-10 known answers and inputs whose correct plan is evident."""
import math

import numpy as np

import oracle
from tests.conftest import load_golden


def _u53(hi, lo):
    return float(((hi << 32) | lo) >> 11) * 2.0 ** -53


def test_draw_uniforms_take_the_published_words():
    """Key 0 and counter (0, 0, 0, 0) is the first published known answer:
    block 0 of row (b, h, r) = (0, 0, 0) takes output words 0 and 1 as
    (high, low), block 1 words 2 and 3."""
    kat = load_golden("philox_kat.yaml")["vectors"][0]
    assert kat["counter"] == [0, 0, 0, 0] and kat["key"] == [0, 0]
    x0, x1, x2, x3 = kat["out"]
    u = oracle.sip_uniforms(0, 0, 0, 0, 2)
    assert u[0] == _u53(x0, x1) and u[1] == _u53(x2, x3)


def test_systematic_uniform_takes_the_published_words():
    """Key (2^32-1, 2^32-1) and counter (2^32-1, r, h, b) with r = h = b =
    2^32-1 is the second published known answer: the row's U is the top 40
    bits of words 0 and 1."""
    kat = load_golden("philox_kat.yaml")["vectors"][1]
    assert kat["counter"] == [0xFFFFFFFF] * 4 and kat["key"] == [0xFFFFFFFF] * 2
    x0, x1 = kat["out"][0], kat["out"][1]
    U = oracle.systematic_uniform(2 ** 64 - 1, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF)
    assert U == ((x0 << 32) | x1) >> 24


def test_plan_rows_are_numbered_batch_head_block():
    """Row (b, h, r) is row (b*H + h)*QB + r: with all of each row's score on
    one block (a different one per row) and a budget of 1, each plan row must
    hold exactly its own block with p = 1 and offset 0."""
    B, H, N, d = 2, 3, 512, 64
    QB, M = (N + 127) // 128, N // 4
    s = np.zeros((B, H, QB, M), np.float32)
    want = {}
    for b in range(B):
        for h in range(H):
            for r in range(QB):
                j = (7 * b + 3 * h + 11 * r) % M
                s[b, h, r, j] = 1.0
                want[(b * H + h) * QB + r] = j
    for sampling in ("poisson", "systematic"):
        plan = oracle.plan_from_scores(s, B, H, N, d, 1, 12345, sampling)
        assert plan.rowptr.tolist() == list(range(B * H * QB + 1))
        assert plan.idx.tolist() == [want[i] for i in range(B * H * QB)]
        assert (plan.p == 1.0).all() and (plan.logw == 0.0).all()


def test_scores_follow_their_head_and_query_block():
    """Each (b, h) has orthogonal key directions; the queries of block r of
    head (b, h) all point at the keys of one KV block f(b, h, r). The score
    row of (b, h, r) must peak at f(b, h, r): heads, batches and query blocks
    are not mixed up, and the softmax runs within the head."""
    B, H, N, d = 2, 2, 256, 64
    QB, M = (N + 127) // 128, N // 4
    rng = np.random.default_rng(0)
    Q = np.zeros((B, H, N, d))
    K = np.zeros((B, H, N, d))
    target = {}
    for b in range(B):
        for h in range(H):
            basis = np.linalg.qr(rng.standard_normal((d, d)))[0]        # orthonormal rows
            # KV block j's four keys are the unit direction basis[j] (M = d)
            for j in range(M):
                K[b, h, 4 * j:4 * j + 4] = basis[j]
            for r in range(QB):
                f = (5 * b + 9 * h + 13 * r + 1) % d                    # a block j < d
                target[(b, h, r)] = f
                Q[b, h, 128 * r:128 * r + 128] = 10.0 * math.sqrt(d) * basis[f] + \
                    0.01 * rng.standard_normal((128, d))
    scores, _, _ = oracle.ibcs_scores(Q, K)
    for (b, h, r), f in target.items():
        row = scores[b, h, r]
        # M = d here: block f is the only one along the queries' direction
        assert int(np.argmax(row)) == f, ((b, h, r), f, int(np.argmax(row)))
        assert row[f] > 0.9
        assert abs(row.sum() - 1.0) < 1e-12
