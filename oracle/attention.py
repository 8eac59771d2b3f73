"""Horvitz-Thompson block-sparse attention and dense attention in fp64.

TEST INFRASTRUCTURE ONLY.

[hamidun, "three techniques in AB-Attention", SIP and kernel paragraphs]: the
chosen 4-token KV blocks are used in their original token order, each chosen
block weighted by 1/p, which is ordinary softmax attention whose logits are
shifted by log(1/p) for every key of that block. Readings: the offset is
added after the 1/sqrt(d) scale; the output is the ratio of the weighted
numerator and normaliser; a row that drew no block returns zeros.
"""
from __future__ import annotations

import math

import numpy as np


def _block_keys(idx: np.ndarray, kv_block: int = 4) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.int64)
    return (idx[:, None] * kv_block + np.arange(kv_block)[None, :]).reshape(-1)


def ht_attention_row(Qr, K, V, idx, logw, kv_block: int = 4):
    """Attention of the queries Qr [n, d] over the chosen KV blocks.

    K, V: [N, d] float64 of the same (batch, head); idx: chosen KV-block
    indices; logw: their fp32 log-weights. Returns [n, d] float64.
    """
    n, d = Qr.shape
    keys = _block_keys(idx, kv_block)
    if keys.size == 0:
        return np.zeros((n, V.shape[1]))
    off = np.repeat(np.asarray(logw, dtype=np.float32).astype(np.float64), kv_block)
    z = Qr @ K[keys].T / math.sqrt(d) + off[None, :]
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e @ V[keys]) / e.sum(axis=1, keepdims=True)


def dense_attention_rows(Qr, K, V):
    """softmax(Qr K^T / sqrt(d)) V for a subset of query rows."""
    d = Qr.shape[1]
    z = Qr @ K.T / math.sqrt(d)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e @ V) / e.sum(axis=1, keepdims=True)


def dense_attention(Q, K, V):
    """Dense softmax attention over [..., N, d] float64 tensors, head by head."""
    out = np.empty(Q.shape[:-1] + (V.shape[-1],))
    for ix in np.ndindex(*Q.shape[:-2]):
        out[ix] = dense_attention_rows(Q[ix], K[ix], V[ix])
    return out


def ht_numerator_denominator(Qr, K, V, idx, p, shift, kv_block: int = 4):
    """Horvitz-Thompson numerator and normaliser with a fixed logit shift.

    N_hat = sum_{j chosen} (1/p_j) sum_{k in j} exp(z_k - shift) v_k and
    D_hat = sum_{j chosen} (1/p_j) sum_{k in j} exp(z_k - shift), where
    z = q . k / sqrt(d) and shift is a per-query constant [n]. Their
    expectations over the Poisson draw are the dense numerator and normaliser.
    """
    n, d = Qr.shape
    keys = _block_keys(idx, kv_block)
    if keys.size == 0:
        return np.zeros((n, V.shape[1])), np.zeros(n)
    wts = np.repeat(1.0 / np.asarray(p, dtype=np.float64), kv_block)
    e = np.exp(Qr @ K[keys].T / math.sqrt(d) - np.asarray(shift)[:, None]) * wts[None, :]
    return e @ V[keys], e.sum(axis=1)
