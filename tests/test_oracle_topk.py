"""Pins of the oracle's Gumbel-Top-K (CPU only).

STAND page, method item 2: adding Gumbel noise to log-probabilities and keeping the indices of
the k largest sums draws k tokens without replacement in one step; the noise is precomputed
and cached. Checks that do not retype the oracle: with zero noise the result is numpy's
ordering of the keys (stable lexsort), k = 1 is the plain Gumbel-max argmax, every row holds k
distinct tokens with non-increasing keys, and over 300 000 noise rows the ordered pair of the
first two tokens follows the sampling-without-replacement law p_a p_b / (1 - p_a).
"""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle


def test_zero_noise_is_sorted_keys():
    # With G = 0 the key is z/T and T > 0, so the k tokens are numpy's stable descending order
    # of z whatever T is, and their keys are z/T.
    rng = np.random.default_rng(0)
    rows, V, k = 40, 257, 17
    z = rng.normal(0, 2, (rows, V)).astype(np.float32)
    z[:, 10:20] = z[:, 10:11]                       # ties on purpose
    T = rng.choice([0.6, 1.0, 1.7], rows).astype(np.float32)
    tok, key, gap = oracle.gumbel_topk(z, T, np.zeros_like(z), k, gaps=True)
    for r in range(rows):
        order = np.lexsort((np.arange(V), -z[r]))[:k]
        assert np.array_equal(tok[r], order)
        np.testing.assert_allclose(key[r], z[r][order].astype(np.float64) / float(T[r]),
                                   rtol=1e-15, atol=0)
        nxt = np.lexsort((np.arange(V), -z[r]))[k]
        np.testing.assert_allclose(gap[r][-1], (float(z[r][order[-1]]) - float(z[r][nxt])) / float(T[r]),
                                   rtol=1e-12, atol=1e-15)


def test_gaps_are_the_distance_to_the_next_rank():
    rng = np.random.default_rng(4)
    rows, V = 20, 50
    z = rng.normal(0, 1, (rows, V)).astype(np.float32)
    g = rng.gumbel(size=(rows, V)).astype(np.float32)
    T = np.full(rows, 0.7, np.float32)
    tok, key, gap = oracle.gumbel_topk(z, T, g, V, gaps=True)   # the whole row: k == V
    assert np.array_equal(gap[:, :-1], key[:, :-1] - key[:, 1:])
    assert np.all(np.isinf(gap[:, -1]))
    assert np.all(gap >= 0)
    for r in range(rows):
        assert sorted(tok[r].tolist()) == list(range(V))
    # the first rank's gap is the bonus draw's top-2 gap
    for r in range(rows):
        idx, g2 = oracle.row_gumbel_argmax(z[r], g[r], 0.7)
        assert idx == tok[r, 0] and g2 == gap[r, 0]


def test_k1_is_gumbel_max():
    rng = np.random.default_rng(1)
    rows, V = 30, 1000
    z = rng.normal(0, 2, (rows, V)).astype(np.float32)
    g = rng.gumbel(size=(rows, V)).astype(np.float32)
    T = np.full(rows, 0.8, np.float32)
    tok, _ = oracle.gumbel_topk(z, T, g, 1)
    for r in range(rows):
        assert tok[r, 0] == oracle.row_gumbel_argmax(z[r], g[r], T=0.8)[0]


def test_distinct_tokens_and_ordered_keys():
    rng = np.random.default_rng(2)
    rows, V, k = 50, 300, 64
    z = rng.normal(0, 1, (rows, V)).astype(np.float32)
    g = rng.gumbel(size=(rows, V)).astype(np.float32)
    tok, key = oracle.gumbel_topk(z, np.ones(rows, np.float32), g, k)
    for r in range(rows):
        assert len(set(tok[r].tolist())) == k
    assert np.all(np.diff(key, axis=1) <= 0)


def test_first_two_follow_sampling_without_replacement():
    rng = np.random.default_rng(3)
    V, rows = 5, 300000
    z = rng.normal(0, 1.0, V).astype(np.float32)
    p = torch.softmax(torch.from_numpy(z.astype(np.float64)), -1).numpy()
    g = rng.gumbel(size=(rows, V)).astype(np.float32)
    tok, _ = oracle.gumbel_topk(np.broadcast_to(z, (rows, V)).copy(), np.ones(rows, np.float32),
                                g, 2)
    pair = tok[:, 0] * V + tok[:, 1]
    counts = np.bincount(pair, minlength=V * V).reshape(V, V)
    expect = p[:, None] * p[None, :] / (1.0 - p[:, None])
    np.fill_diagonal(expect, 0.0)
    mask = ~np.eye(V, dtype=bool)
    assert counts[~mask].sum() == 0                  # never the same token twice
    chi2, pval = stats.chisquare(counts[mask], rows * expect[mask])
    assert pval > 1e-3, (chi2, pval)
    # sampling WITH replacement (p_a p_b) would be rejected
    alt = p[:, None] * p[None, :]
    alt = alt[mask] / alt[mask].sum()
    _, pval_alt = stats.chisquare(counts[mask], rows * alt)
    assert pval_alt < 1e-6
