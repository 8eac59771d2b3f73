"""Pins of the oracle's HT attention and dense attention (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.conftest import load_golden


def _sdpa(Q, K, V):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None])[0].numpy()


def test_dense_matches_library_attention():
    rng = np.random.default_rng(0)
    Q, K, V = (rng.standard_normal((2, 3, 96, 16)) * 2 for _ in range(3))
    out = oracle.dense_attention(Q, K, V)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V)).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_dense_special_cases():
    rng = np.random.default_rng(1)
    V = rng.standard_normal((12, 4))
    # identical keys: every query averages V
    out = oracle.dense_attention_rows(rng.standard_normal((3, 4)), np.ones((12, 4)), V)
    np.testing.assert_allclose(out, np.tile(V.mean(0), (3, 1)), atol=1e-14)
    # one key: output is its value
    out = oracle.dense_attention_rows(rng.standard_normal((2, 4)), rng.standard_normal((1, 4)), V[:1])
    np.testing.assert_allclose(out, np.tile(V[0], (2, 1)), atol=1e-15)


@pytest.mark.parametrize("i", range(2))
def test_ht_hand_examples(i):
    g = load_golden("ht_examples.yaml")["cases"][i]
    Q = np.zeros((1, 1))
    K = np.zeros((8, 1))
    V = np.array([g["v_block0"]] * 4 + [g["v_block1"]] * 4)[:, None]
    p = np.array(g["p"])
    logw = np.where(p == 1, 0.0, -np.log(p)).astype(np.float32)
    out = oracle.ht_attention_row(Q, K, V, np.array([0, 1]), logw)
    np.testing.assert_allclose(out[0, 0], g["out"], rtol=1e-7)


def test_ht_offset_equals_duplicated_keys():
    # a block with p = 1/4 counts four times: the same as physically
    # repeating its 4 keys four times in a library attention call
    rng = np.random.default_rng(2)
    N, d = 64, 8
    Q, K, V = (rng.standard_normal((n, d)) for n in (5, N, N))
    idx = np.array([1, 4, 9, 15])
    p = np.array([1.0, 0.25, 1.0, 0.25])
    logw = np.where(p == 1, 0.0, -np.log(p)).astype(np.float32)
    out = oracle.ht_attention_row(Q, K, V, idx, logw)
    keys = []
    for j, pj in zip(idx, p):
        keys += list(range(4 * j, 4 * j + 4)) * int(round(1 / pj))
    ref = _sdpa(Q, K[keys], V[keys])
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-6)


def test_ht_uniform_offsets_cancel():
    rng = np.random.default_rng(3)
    Q, K, V = (rng.standard_normal((n, 8)) for n in (4, 40, 40))
    idx = np.array([0, 3, 7, 9])
    out = oracle.ht_attention_row(Q, K, V, idx, np.full(4, 2.5, np.float32))
    keys = (idx[:, None] * 4 + np.arange(4)).ravel()
    np.testing.assert_allclose(out, _sdpa(Q, K[keys], V[keys]), atol=1e-13)
    # no block drawn: the row is zero
    assert not oracle.ht_attention_row(Q, K, V, np.zeros(0, int), np.zeros(0, np.float32)).any()


def test_plan_full_budget_equals_dense():
    q, k, v = synth.iid_qkv(1, 2, 1024, 64, seed=0)
    Q, K, V = (x.astype(np.float64) for x in (q, k, v))
    M = 256
    plan = oracle.build_plan(Q, K, budget=M, seed=synth.sip_seed(0))
    assert (plan.p == 1).all() and (plan.logw == 0).all()
    np.testing.assert_array_equal(np.diff(plan.rowptr), M)
    out = oracle.plan_attention(Q, K, V, plan)
    np.testing.assert_allclose(out, oracle.dense_attention(Q, K, V), rtol=0, atol=1e-12)


def test_ht_numerator_and_normaliser_unbiased():
    # Monte-Carlo over seeds on a tiny workload: the means of the HT
    # numerator and normaliser approach the dense ones within 5 standard
    # errors of the closed-form Poisson variance sum_j (1-p_j)/p_j a_j^2
    q, k, v = synth.iid_qkv(1, 1, 256, 16, seed=3)
    Q, K, V = (x[0, 0].astype(np.float64) for x in (q, k, v))
    kbar = oracle.mean_keys(K)
    s, _, _ = oracle.ibcs_row(Q[:128], kbar)
    p = oracle.sip_probabilities(s.astype(np.float32), 16)
    Qr = Q[:4]
    z = Qr @ K.T / math.sqrt(16)
    shift = z.max(1)
    e = np.exp(z - shift[:, None])                            # [n, N]
    a_den = e.reshape(4, 64, 4).sum(2)                        # per block
    a_num = np.einsum("nk,kd->nkd", e, V).reshape(4, 64, 4, 16).sum(2)
    dense_num, dense_den = e @ V, e.sum(1)
    S = 3000
    acc_num = np.zeros_like(dense_num)
    acc_den = np.zeros_like(dense_den)
    for seed in range(S):
        idx, logw, pk = oracle.sip_draw_row(p, seed, 0, 0, 0)
        n_hat, d_hat = oracle.ht_numerator_denominator(Qr, K, V, idx, pk, shift)
        acc_num += n_hat
        acc_den += d_hat
    w = (1 - p) / p
    var_den = (a_den ** 2 * w[None, :]).sum(1)
    var_num = (a_num ** 2 * w[None, :, None]).sum(1)
    assert (np.abs(acc_den / S - dense_den) <= 5 * np.sqrt(var_den / S) + 1e-12).all()
    assert (np.abs(acc_num / S - dense_num) <= 5 * np.sqrt(var_num / S) + 1e-12).all()
    # a plausible slip (dropping the 1/p weights) is caught by the same test
    biased = np.zeros_like(dense_den)
    for seed in range(200):
        idx, _, pk = oracle.sip_draw_row(p, seed, 0, 0, 0)
        biased += oracle.ht_numerator_denominator(Qr, K, V, idx, np.ones_like(pk), shift)[1]
    assert (np.abs(biased / 200 - dense_den) > 5 * np.sqrt(var_den / 200)).any()
