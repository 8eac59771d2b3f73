"""CPU checks of the selection study's arithmetic in bench.py (retained
attention mass, recall of the exact top-K, top-K and 128-token plans, true
block masses): hand examples and the properties that must hold for any
input."""
import math

import numpy as np
import pytest

import bench


def test_retained_mass_hand_example():
    mass = np.array([[0.5, 0.3, 0.2], [0.1, 0.1, 0.8]])
    rowptr = np.array([0, 2, 3])
    idx = np.array([0, 1, 2])
    np.testing.assert_allclose(bench.retained_mass(mass, rowptr, idx), [0.8, 0.8])
    # an empty row retains nothing
    np.testing.assert_allclose(bench.retained_mass(mass, np.array([0, 0, 1]), np.array([2])),
                               [0.0, 0.8])


def test_exact_topk_retains_the_most_and_full_budget_retains_all():
    rng = np.random.default_rng(3)
    rows, M, K = 12, 64, 9
    mass = rng.dirichlet(np.full(M, 0.3), size=rows)
    exact = bench.retained_mass(mass, *bench.topk_plan(mass, K)[:2])
    for trial in range(20):
        other = rng.random((rows, M))
        got = bench.retained_mass(mass, *bench.topk_plan(other, K)[:2])
        assert (exact >= got - 1e-15).all()
    full = bench.retained_mass(mass, *bench.topk_plan(mass, M)[:2])
    np.testing.assert_allclose(full, 1.0, atol=1e-12)


def test_topk_plan_and_recall():
    score = np.array([[0.1, 0.4, 0.3, 0.2], [0.9, 0.0, 0.05, 0.05]])
    rowptr, idx, logw, p = bench.topk_plan(score, 2)
    assert rowptr.tolist() == [0, 2, 4]
    assert idx.tolist() == [1, 2, 0, 2] or idx.tolist() == [1, 2, 0, 3]
    assert (logw == 0).all() and (p == 1).all()
    ref = (np.array([0, 2, 4]), np.array([1, 3, 0, 1]))
    rec = bench.recall(rowptr, idx, *ref)
    assert rec[0] == 0.5 and rec[1] == 0.5
    assert bench.recall(*ref, *ref).tolist() == [1.0, 1.0]


def test_coarse_plan_takes_whole_groups():
    rng = np.random.default_rng(4)
    score = rng.random((3, 256))
    rowptr, idx, _, _ = bench.coarse_plan(score, 70, group=32)   # 70 // 32 = 2 groups
    assert np.diff(rowptr).tolist() == [64, 64, 64]
    for r in range(3):
        g = idx[rowptr[r]:rowptr[r + 1]].reshape(2, 32)
        assert (g % 32 == np.arange(32)).all() and (g[:, 0] % 32 == 0).all()
        sums = score[r].reshape(8, 32).sum(axis=1)
        assert set(g[:, 0] // 32) == set(np.argsort(-sums)[:2])


def test_block_masses_are_softmax_sums():
    rng = np.random.default_rng(5)
    Q, K = rng.standard_normal((5, 8)), rng.standard_normal((16, 8))
    m = bench.block_masses(Q, K)
    assert m.shape == (4,) and abs(m.sum() - 1.0) < 1e-12
    z = np.exp(Q @ K.T / math.sqrt(8))
    z /= z.sum(axis=1, keepdims=True)
    want = np.array([z[:, 4 * j:4 * j + 4].sum(axis=1).mean() for j in range(4)])
    np.testing.assert_allclose(m, want, atol=1e-14)
