"""Whole-round law pin of the oracle (CPU only).

SMC-SD trades exact sampling for speed; its approximation error shrinks as the number of
particles grows ("Faster LLM Inference via Sequential Monte Carlo", section 3: approximate
rather than exact sampling, bias and MSE bounds that fall with N). Reading: bias O(1/N).

Toy model, V = 4 tokens, K = 2 drafted tokens: target and draft are two-step autoregressive
tables p(x1) p(x2|x1), q(x1) q(x2|x1) built from seeded logits; each particle's second row
is the conditional row of its own first token. The law of one particle picked from the
resampled population is L_N(s) = E[sum_i W_i 1{s_i = s}] (systematic resampling is unbiased,
E_u[o_i] = N W_i, pinned separately by exact integration over u).

  * N <= 4: L_N by enumerating all 16^N particle sets through the oracle's round;
    L_1 = q exactly, sum L_N = 1, TV(L_N, p) strictly decreasing.
  * N up to 1024: L_N(s) = N q(s) E[w(s) / (w(s) + S)], S the total weight of N-1 i.i.d.
    particles, averaged over multinomial counts with the oracle's per-sequence weights;
    N * TV(L_N, p) stays within a narrow band (bias O(1/N)) while TV itself falls 100x.
A weight of q/p instead of p/q, a dropped position, or a wrong normalisation moves L_N away
from p and fails these checks.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle

V, K = 4, 2


def _toy(seed=21):
    rng = np.random.default_rng(seed)
    zp0 = rng.normal(0, 1.5, V).astype(np.float32)
    zp1 = rng.normal(0, 1.5, (V, V)).astype(np.float32)
    zq0 = (zp0 + rng.normal(0, 1.0, V)).astype(np.float32)
    zq1 = (zp1 + rng.normal(0, 1.0, (V, V))).astype(np.float32)
    sm = lambda z: torch.softmax(torch.from_numpy(z.astype(np.float64)), -1).numpy()
    p = (sm(zp0)[:, None] * sm(zp1)).ravel()           # p(s), s = 4*x1 + x2
    q = (sm(zq0)[:, None] * sm(zq1)).ravel()
    return (zp0, zp1, zq0, zq1), p, q


def _round_inputs(tables, seqs):
    zp0, zp1, zq0, zq1 = tables
    R, N = seqs.shape
    x1, x2 = seqs // V, seqs % V
    tgt = np.zeros((R, N, K + 1, V), np.float32)
    dft = np.zeros((R, N, K, V), np.float32)
    tgt[:, :, 0] = zp0
    tgt[:, :, 1] = zp1[x1]
    dft[:, :, 0] = zq0
    dft[:, :, 1] = zq1[x1]
    return dict(target=tgt, draft=dft, tokens=np.stack([x1, x2], -1).astype(np.int32),
                temperature=np.ones(R, np.float32), gumbel=np.zeros((R, N, V), np.float32),
                uniform=np.zeros(R, np.float32),
                log_weights=np.full((R, N), -math.log(N), np.float32))


def _tv(a, b):
    return 0.5 * np.abs(a - b).sum()


def test_exact_law_small_n():
    tables, p, q = _toy()
    tvs = []
    for N in range(1, 5):
        seqs = np.array(list(itertools.product(range(V * V), repeat=N)))
        out = oracle.round(_round_inputs(tables, seqs), mode="never")
        W = np.exp(out["log_weights"])
        prob = np.prod(q[seqs], axis=1)
        L = np.zeros(V * V)
        for i in range(N):
            np.add.at(L, seqs[:, i], prob * W[:, i])
        assert L.sum() == pytest.approx(1.0, abs=1e-12)
        if N == 1:
            assert np.allclose(L, q, atol=1e-14)        # one particle: the draft's own law
        tvs.append(_tv(L, p))
    assert all(a > b for a, b in zip(tvs, tvs[1:])), tvs
    assert tvs[-1] < 0.5 * tvs[0]


def test_per_sequence_weights_are_target_over_draft():
    tables, p, q = _toy()
    seqs = np.arange(V * V)[None, :]
    out = oracle.round(_round_inputs(tables, seqs), mode="never")
    w = np.exp(out["log_w_incr"][0])
    assert np.allclose(w, p / q, rtol=1e-12)


def test_bias_shrinks_as_one_over_n():
    tables, p, q = _toy()
    seqs = np.arange(V * V)[None, :]
    w = np.exp(oracle.round(_round_inputs(tables, seqs), mode="never")["log_w_incr"][0])
    rng = np.random.default_rng(5)
    scaled = []
    tvs = []
    for N in (16, 64, 256, 1024):
        n = rng.multinomial(N - 1, q, size=200000)
        S = n @ w
        L = N * q * np.mean(w[None, :] / (w[None, :] + S[:, None]), axis=0)
        tvs.append(_tv(L, p))
        scaled.append(N * tvs[-1])
    assert tvs[-1] < tvs[0] / 30                        # TV keeps falling with N
    assert max(scaled) / min(scaled) < 1.25, scaled     # ... like c / N
