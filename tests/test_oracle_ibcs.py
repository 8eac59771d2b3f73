"""Pins of the oracle's mean keys, k-means and IBCS scores (CPU only).

Each check ties the oracle to something other than itself: hand-worked
fixtures, closed forms, invariants, or a reduction to a library softmax.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle
from tests.conftest import load_golden


def test_mean_keys_hand_example():
    g = load_golden("ibcs_examples.yaml")["mean_keys"]
    K = np.array(g["keys"], dtype=np.float64)
    np.testing.assert_array_equal(oracle.mean_keys(K), np.array(g["kbar"], dtype=np.float64))


def test_mean_keys_constant_blocks_and_total():
    rng = np.random.default_rng(1)
    consts = rng.standard_normal((3, 6, 5))                   # [H, M, d]
    K = np.repeat(consts, 4, axis=1)                          # every block constant
    np.testing.assert_allclose(oracle.mean_keys(K), consts, rtol=0, atol=1e-15)
    K2 = rng.standard_normal((2, 16, 7))
    # four times the sum of the averaged keys equals the sum of all keys
    np.testing.assert_allclose(4 * oracle.mean_keys(K2).sum(1), K2.sum(1), atol=1e-12)
    with pytest.raises(ValueError):
        oracle.mean_keys(np.zeros((6, 2)))


@pytest.mark.parametrize("case", range(4))
def test_kmeans_hand_examples(case):
    g = load_golden("ibcs_examples.yaml")["kmeans"][case]
    Q = np.array(g["queries"], dtype=np.float64)
    c, w, a = oracle.kmeans_block(Q, g["clusters"], g["iters"])
    np.testing.assert_allclose(c, np.array(g["centroids"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(w, np.array(g["weights"]), rtol=0, atol=1e-15)
    np.testing.assert_array_equal(a, np.array(g["assign"]))


def _video_block(seed, n=128, d=32):
    rng = np.random.default_rng(seed)
    f = np.sin(np.linspace(0, 3, n)[:, None] * rng.integers(1, 3, d)[None, :] + rng.uniform(0, 6, d))
    return 0.5 * rng.standard_normal((n, d)) + 2 * f


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("n", [128, 80, 16, 5, 1])
def test_kmeans_invariants(seed, n):
    Q = _video_block(seed, n=n)
    c, w, a = oracle.kmeans_block(Q, 8, 4)
    # weights are shares of the block's queries: they sum to one, and
    # k * n are the member counts
    assert abs(w.sum() - 1.0) < 1e-15
    np.testing.assert_array_equal(np.round(w * n).astype(int), np.bincount(a, minlength=8))
    # every non-empty centroid is the mean of its members
    for m in range(8):
        if w[m] > 0:
            np.testing.assert_allclose(c[m], Q[a == m].mean(0), atol=1e-13)
    # the weighted centroids reproduce the block's mean query
    np.testing.assert_allclose(w @ c, Q.mean(0), atol=1e-12)
    assert (w[min(8, n):] == 0).all()


def test_kmeans_single_cluster_is_block_mean():
    Q = _video_block(3)
    c, w, a = oracle.kmeans_block(Q, 1, 4)
    np.testing.assert_allclose(c[0], Q.mean(0), atol=1e-13)
    assert w[0] == 1.0 and (a == 0).all()


def test_kmeans_one_cluster_per_query():
    Q = _video_block(4, n=8)
    c, w, a = oracle.kmeans_block(Q, 8, 4)
    np.testing.assert_array_equal(c, Q)
    np.testing.assert_array_equal(a, np.arange(8))
    np.testing.assert_array_equal(w, np.full(8, 1 / 8))


def test_kmeans_recovers_planted_clusters():
    rng = np.random.default_rng(5)
    centers = rng.standard_normal((8, 16)) * 20.0
    Q = np.repeat(centers, 16, axis=0) + rng.standard_normal((128, 16)) * 0.1
    c, w, a = oracle.kmeans_block(Q, 8, 4)
    np.testing.assert_array_equal(a, np.repeat(np.arange(8), 16))
    for m in range(8):
        np.testing.assert_allclose(c[m], Q[16 * m:16 * m + 16].mean(0), atol=1e-12)
    np.testing.assert_array_equal(w, np.full(8, 1 / 8))


def test_scores_hand_example():
    g = load_golden("ibcs_examples.yaml")["scores"][0]
    s = oracle.ibcs_scores_row(np.array(g["centroids"]), np.array(g["weights"]),
                               np.array(g["kbar"]), d=1)
    np.testing.assert_allclose(s, g["scores"], rtol=0, atol=1e-15)


def _head(seed, N=512, d=32):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((N, d)) * 1.5
    K = rng.standard_normal((N, d)) * 1.5
    return Q, K


def test_scores_single_cluster_is_block_mean_softmax():
    # one cluster: the score is the softmax of the block's mean query against
    # the averaged keys (block-mean scoring)
    Q, K = _head(6)
    kbar = oracle.mean_keys(K)
    s, c, w = oracle.ibcs_row(Q[:128], kbar, n_clusters=1, iters=3)
    ref = softmax(Q[:128].mean(0) @ kbar.T / math.sqrt(32))
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-15)


def test_scores_cluster_per_query_is_mean_of_query_softmaxes():
    Q, K = _head(7)
    kbar = oracle.mean_keys(K)
    Qr = Q[:8]
    s, _, _ = oracle.ibcs_row(Qr, kbar, n_clusters=8, iters=2)
    ref = softmax(Qr @ kbar.T / math.sqrt(32), axis=1).mean(0)
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-15)
    # the same through the library attention on the CPU: attention weights of
    # each query on the averaged keys, via scaled_dot_product_attention with
    # an identity value matrix
    att = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Qr)[None], torch.from_numpy(kbar)[None],
        torch.eye(kbar.shape[0], dtype=torch.float64)[None])[0].numpy()
    np.testing.assert_allclose(s, att.mean(0), rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("n", [128, 80])
def test_scores_invariants(n):
    Q, K = _head(8)
    kbar = oracle.mean_keys(K)
    s, c, w = oracle.ibcs_row(Q[:n], kbar)
    assert (s >= 0).all() and abs(s.sum() - 1.0) < 1e-12
    # shifting every key by one vector shifts each centroid's logits by a
    # constant, which the softmax ignores
    shift = np.random.default_rng(9).standard_normal(32)
    s2 = oracle.ibcs_scores_row(c, w, kbar + shift, 32)
    np.testing.assert_allclose(s2, s, rtol=1e-9, atol=1e-15)
    # permuting KV blocks permutes the scores
    perm = np.random.default_rng(10).permutation(kbar.shape[0])
    s3 = oracle.ibcs_scores_row(c, w, kbar[perm], 32)
    np.testing.assert_allclose(s3, s[perm], rtol=1e-12, atol=1e-16)


def test_full_scores_shapes_and_rows():
    rng = np.random.default_rng(11)
    Q = rng.standard_normal((1, 2, 200, 16))
    K = rng.standard_normal((1, 2, 200, 16))
    S, C, W = oracle.ibcs_scores(Q, K)
    assert S.shape == (1, 2, 2, 50) and C.shape == (1, 2, 2, 8, 16) and W.shape == (1, 2, 2, 8)
    np.testing.assert_allclose(S.sum(-1), 1.0, atol=1e-12)
    # the partial last block (72 queries) is clustered on its own queries only
    c, w, _ = oracle.kmeans_block(Q[0, 1, 128:200], 8, 4)
    np.testing.assert_array_equal(C[0, 1, 1], c)


def test_kmeans_tie_variants_hand_example():
    """Queries 0, 2, 1 on a line with C = 2 and T = 1: the initial centroids
    are q[0] = 0 and q[1] = 2, and q[2] = 1 is exactly as far from both. The
    rule gives it to cluster 0 (weights 2/3, 1/3; centroids 0.5 and 2); the
    other side of the tie gives it to cluster 1 (weights 1/3, 2/3; centroids
    0 and 1.5)."""
    Q = np.array([[0.0], [2.0], [1.0]])
    var = oracle.kmeans_tie_variants(Q, 2, 1)
    assert len(var) == 2
    (c0, w0, ov0), (c1, w1, ov1) = var
    assert ov0 == {} and ov1 == {(0, 2): 1}
    np.testing.assert_array_equal(w0, [2 / 3, 1 / 3])
    np.testing.assert_array_equal(c0[:, 0], [0.5, 2.0])
    np.testing.assert_array_equal(w1, [1 / 3, 2 / 3])
    np.testing.assert_array_equal(c1[:, 0], [0.0, 1.5])
    # the plain result is kmeans_block's
    c, w, _ = oracle.kmeans_block(Q, 2, 1)
    np.testing.assert_array_equal(c, c0)
    np.testing.assert_array_equal(w, w0)
    # well-separated queries have no near-tie: one variant only
    Qs = _video_block(3)
    assert len(oracle.kmeans_tie_variants(Qs, 8, 4)) == 1


def test_kmeans_tie_variants_two_ties_branch_in_order():
    """Two exact ties in the first iteration (T = 1) give four results: the
    plain one and each combination of the other sides."""
    Q = np.array([[0.0], [1.0], [2.0], [1.0]])     # initial centroids q[0], q[2]
    var = oracle.kmeans_tie_variants(Q, 2, 1)
    assert sorted(tuple(sorted(v[2].items())) for v in var) == [
        (), (((0, 1), 1),), (((0, 1), 1), ((0, 3), 1)), (((0, 3), 1),)]
    counts = sorted(tuple(np.round(v[1] * 4).astype(int)) for v in var)
    assert counts == [(1, 3), (2, 2), (2, 2), (3, 1)]
